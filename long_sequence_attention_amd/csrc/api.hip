// C ABI of the library: argument validation (before any HIP call), launch
// geometry and status codes. Declarations and contracts: include/dit_attn.h.
#include "dit_attn.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"

// Workspace of dit_attn_fwd_noalloc: one copy per GPU the library runs on,
// held until the process ends. Host code uses only the device address
// that hipGetSymbolAddress returns for it (scratch_ptr below), never the
// array's own name, which on the host is only a stand-in.
static __device__ __align__(256) unsigned char scratch[DIT_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[1024];

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DIT_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(DIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Resolve a (b, h, s) stride triple; all zeros means dense [B, H, S, d].
void resolve_strides(const int64_t in[3], int H, int S, int d, int64_t out[3]) {
  if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
    out[0] = (int64_t)H * S * d;
    out[1] = (int64_t)S * d;
    out[2] = d;
  } else {
    out[0] = in[0];
    out[1] = in[1];
    out[2] = in[2];
  }
}

int check_strides(const char *name, const int64_t st[3]) {
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(DIT_ERR_UNSUPPORTED, "%s stride[%d] = %lld: negative strides are not supported", name, i, (long long)st[i]);
    if (st[i] % 8 != 0)
      return fail(DIT_ERR_UNSUPPORTED, "%s stride[%d] = %lld: strides must be multiples of 8 elements", name, i, (long long)st[i]);
  }
  return DIT_OK;
}

size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

int validate_attn(const dit_attn_desc *d, float *scale_out) {
  if (d == nullptr) return fail(DIT_ERR_INVALID, "desc is NULL");
  if (d->B < 1 || d->H < 1) return fail(DIT_ERR_INVALID, "B and H must be >= 1 (B=%d, H=%d)", d->B, d->H);
  if (d->d <= 0 || (d->d % 2) != 0) return fail(DIT_ERR_INVALID, "head dim d=%d must be positive and even", d->d);
  if (d->d != 64 && d->d != 128) return fail(DIT_ERR_UNSUPPORTED, "head dim d=%d: kernels exist for d in {64, 128}", d->d);
  if (d->s_q < 0 || d->s_kv < 0) return fail(DIT_ERR_INVALID, "s_q and s_kv must be >= 0");
  if (d->q_seg_len < 0 || d->kv_seg_len < 0) return fail(DIT_ERR_INVALID, "segment lengths must be >= 0");
  if (d->q_seg_len > 0 && d->s_q % d->q_seg_len != 0)
    return fail(DIT_ERR_INVALID, "s_q=%d is not a multiple of q_seg_len=%d", d->s_q, d->q_seg_len);
  if (d->kv_seg_len > 0 && d->s_kv % d->kv_seg_len != 0)
    return fail(DIT_ERR_INVALID, "s_kv=%d is not a multiple of kv_seg_len=%d", d->s_kv, d->kv_seg_len);
  const int q_lim = d->q_seg_len > 0 ? d->q_seg_len : d->s_q;
  const int kv_lim = d->kv_seg_len > 0 ? d->kv_seg_len : d->s_kv;
  if (d->q_valid < 0 || d->q_valid > q_lim)
    return fail(DIT_ERR_INVALID, "q_valid=%d must lie in [0, %d] (s_q or q_seg_len)", d->q_valid, q_lim);
  if (d->kv_valid < 0 || d->kv_valid > kv_lim)
    return fail(DIT_ERR_INVALID, "kv_valid=%d must lie in [0, %d] (s_kv or kv_seg_len)", d->kv_valid, kv_lim);
  if (d->kv_seg_len > 0 && d->kv_seg_len % dit::kAttnBlockN != 0)
    return fail(DIT_ERR_UNSUPPORTED, "kv_seg_len=%d must be a multiple of the %d-row key tile", d->kv_seg_len,
                dit::kAttnBlockN);
  if (d->fixed_m < 0 || d->fixed_m > 2) return fail(DIT_ERR_INVALID, "fixed_m=%d must be 0, 1 or 2", d->fixed_m);
  if (d->ws_counters_zero != 0 && d->ws_counters_zero != 1)
    return fail(DIT_ERR_INVALID, "ws_counters_zero=%d must be 0 or 1", d->ws_counters_zero);
  if (d->o_dtype != DIT_BF16 && d->o_dtype != DIT_F32) return fail(DIT_ERR_INVALID, "o_dtype=%d is not a dit_dtype", d->o_dtype);
  if (d->s_q > 0 && (d->q == nullptr || d->o == nullptr)) return fail(DIT_ERR_INVALID, "q and o must be non-NULL when s_q > 0");
  if (d->kv_valid > 0 && (d->k == nullptr || d->v == nullptr))
    return fail(DIT_ERR_INVALID, "k and v must be non-NULL when kv_valid > 0");
  if ((d->cos_q == nullptr) != (d->sin_q == nullptr)) return fail(DIT_ERR_INVALID, "cos_q and sin_q must both be given or both be NULL");
  if ((d->cos_k == nullptr) != (d->sin_k == nullptr)) return fail(DIT_ERR_INVALID, "cos_k and sin_k must both be given or both be NULL");
  float scale = d->sm_scale;
  if (scale == 0.0f) scale = 1.0f / std::sqrt((float)d->d);
  if (!std::isfinite(scale) || scale < 0.0f) return fail(DIT_ERR_INVALID, "sm_scale=%g must be finite and positive", (double)d->sm_scale);
  const int64_t nq = ((int64_t)d->s_q + dit::kAttnBlockM - 1) / dit::kAttnBlockM;
  if (nq * d->H * d->B > 0x7fffffffLL) return fail(DIT_ERR_UNSUPPORTED, "too many query tiles for one launch");
  const bool prep_q = d->cos_q != nullptr || d->q_norm_w != nullptr;
  const bool prep_k = d->cos_k != nullptr || d->k_norm_w != nullptr;
  if ((d->q_norm_w != nullptr || d->k_norm_w != nullptr) && (!std::isfinite(d->norm_eps) || d->norm_eps < 0.0f))
    return fail(DIT_ERR_INVALID, "norm_eps=%g must be finite and >= 0", (double)d->norm_eps);
  if ((prep_q || prep_k) && (int64_t)d->B * d->H > 4LL * 65535)
    return fail(DIT_ERR_UNSUPPORTED, "rotation / normalisation needs B * H <= 262140 (one grid plane per four heads)");
  const void *ptrs[] = {d->q, d->k, d->v, d->o, d->cos_q, d->sin_q, d->cos_k, d->sin_k, d->q_norm_w, d->k_norm_w};
  for (const void *p : ptrs)
    if (p != nullptr && !aligned16(p)) return fail(DIT_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  if (d->lse != nullptr && (reinterpret_cast<uintptr_t>(d->lse) & 3u)) return fail(DIT_ERR_INVALID, "lse must be 4-byte aligned");
  int64_t st[3];
  int rc;
  resolve_strides(d->q_stride, d->H, d->s_q, d->d, st);
  if ((rc = check_strides("q", st)) != DIT_OK) return rc;
  resolve_strides(d->k_stride, d->H, d->s_kv, d->d, st);
  if ((rc = check_strides("k", st)) != DIT_OK) return rc;
  resolve_strides(d->v_stride, d->H, d->s_kv, d->d, st);
  if ((rc = check_strides("v", st)) != DIT_OK) return rc;
  resolve_strides(d->o_stride, d->H, d->s_q, d->d, st);
  if ((rc = check_strides("o", st)) != DIT_OK) return rc;
  // K/V rows are fetched through 32-bit buffer views of one head's rows
  int64_t kst[3], vst[3];
  resolve_strides(d->k_stride, d->H, d->s_kv, d->d, kst);
  resolve_strides(d->v_stride, d->H, d->s_kv, d->d, vst);
  if ((int64_t)d->kv_valid * kst[2] * 2 > 0x7fffffffLL || (int64_t)d->kv_valid * vst[2] * 2 > 0x7fffffffLL)
    return fail(DIT_ERR_UNSUPPORTED, "kv_valid * row stride of K or V exceeds 2 GiB for one head");
  *scale_out = scale;
  return DIT_OK;
}

// Launch plan of one dit_attn_fwd call: Q / K pre-pass and schedule, and where
// their scratch lives inside the caller's workspace.
struct AttnPlan {
  size_t k_bytes = 0;       // prepared (normalised / rotated) K, dense [B, H, s_kv, d] bf16
  size_t q_bytes = 0;       // prepared Q, dense [B, H, s_q, d] bf16 (after K)
  int sk_grid = 0;          // split-schedule workgroups (0 = one workgroup per q-tile)
  int sk_main = 0, sk_kc = 0;
  int dyn_grid = 0;         // dynamic placement: workgroups (q-tiles plus spares; 0 = off)
  int dyn_static = 0;       // ... of which the first wave, placed by index
  size_t part_o_off = 0, part_l_off = 0, count_off = 0;
  int64_t n_counts = 0;
  // fixed-m statistics (fm = false: online softmax)
  bool fm = false;
  int n_chunks = 0, n_real = 0;
  size_t fm_part_off = 0, fm_kbar_off = 0, fm_r2_off = 0, fm_m_off = 0, fm_ok_off = 0;
  size_t total = 0;
};

constexpr int kBlockM = dit::kAttnBlockM, kBlockN = dit::kAttnBlockN, kThreads = dit::kAttnThreads;
constexpr int64_t kDynMinWaves = 4;   // AUTO's dynamic placement: from this many waves of q-tiles

// Split schedule for nq q-tiles of nk key tiles on `cus` compute units
// (one workgroup per CU). Two shapes, modelled in tile-steps, the cheaper
// one taken. A workgroup whose run of units touches a q-tile it does not
// finish pays kPieceCost tile-steps for that piece (its Q load and partial
// store); a run of u units over q-tiles of t units touches at most
// ceil(u / t) + 1 of them, and a q-tile of t units split into runs of u is
// in at most ceil(t / u) + 1 pieces, which its last piece merges at
// kMergeCost tile-steps each.
//  - hybrid (nq < cus): nq main workgroups run keys [0, kc) of their q-tile
//    and up to cus - nq helpers split the nq * (nk - kc) tail units into
//    equal contiguous runs; the tail length is the one that minimises the
//    larger of kc and the busiest helper's units plus piece costs, plus the
//    merge;
//  - plain Stream-K: min(nq * nk, cus) workgroups split all units evenly.
constexpr int64_t kPieceCost = 4, kMergeCost = 1;
struct SplitPlan {
  int grid = 0, main = 0, kc = 0;
};
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
SplitPlan split_plan(int64_t nq, int64_t nk, int64_t cus) {
  SplitPlan sp;
  const int64_t units = nq * nk;
  const int64_t grid = units < cus ? units : cus;
  const int64_t per_sk = ceil_div(units, grid);
  int64_t best = per_sk + (ceil_div(per_sk, nk) + 1) * kPieceCost + (ceil_div(nk, per_sk) + 1) * kMergeCost;
  sp.grid = (int)grid;
  if (nq < cus) {
    int64_t hb = -1, ht = 0, hh = 0;   // the best hybrid: cost, tail length, helpers
    for (int64_t t = 1; t < nk; ++t) {
      const int64_t tail = nq * t;
      const int64_t h = cus - nq < tail ? cus - nq : tail;
      const int64_t per = ceil_div(tail, h);   // the busiest helper's units
      const int64_t helper = per + (ceil_div(per, t) + 1) * kPieceCost;
      const int64_t cost = (nk - t > helper ? nk - t : helper) + (ceil_div(t, per) + 2) * kMergeCost;
      if (hb < 0 || cost < hb) {   // ties keep the shorter tail (fewer pieces)
        hb = cost;
        ht = t;
        hh = h;
      }
    }
    if (hb >= 0 && hb <= best) {   // ties go to the hybrid (fewer pieces per q-tile)
      sp.grid = (int)(nq + hh);
      sp.main = (int)nq;
      sp.kc = (int)(nk - ht);
    }
  }
  return sp;
}

// Compute units of the current device, or 0 when it cannot be queried (AUTO
// then keeps one workgroup per q-tile). Cached per device id.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}
// fixed_m = 0 (AUTO) takes the fixed-m softmax where a head has at least
// kFixedMMinKeys real keys: its statistics passes (a few us) are then a
// small part of the call and the loop without a running maximum wins (Wan
// 720p, 75,600 keys: 23,984 against 24,311 us); on shorter key ranges the
// passes cost more than they save (Wan 480p: 139.7 against 118.2 us).
constexpr int64_t kFixedMMinKeys = 32768;
bool use_fixed_m(const dit_attn_desc *d) {
  if (d->fixed_m == 1) return true;
  if (d->fixed_m == 2) return false;
  const int64_t real_keys = d->kv_seg_len > 0 ? (int64_t)(d->s_kv / d->kv_seg_len) * d->kv_valid : d->kv_valid;
  return real_keys >= kFixedMMinKeys;
}

int plan_attn(const dit_attn_desc *d, AttnPlan *pl) {
  AttnPlan p;
  const bool fm = use_fixed_m(d);
  if ((d->cos_k != nullptr || d->k_norm_w != nullptr) && d->kv_valid > 0)
    p.k_bytes = round_up((size_t)d->B * d->H * (size_t)d->s_kv * d->d * 2, 256);
  if ((d->cos_q != nullptr || d->q_norm_w != nullptr) && d->kv_valid > 0)
    p.q_bytes = round_up((size_t)d->B * d->H * (size_t)d->s_q * d->d * 2, 256);
  const int64_t nq = (int64_t)d->B * d->H * ((d->s_q + kBlockM - 1) / kBlockM);
  const int64_t nk = (d->kv_valid + kBlockN - 1) / kBlockN;
  if (d->schedule < DIT_SCHED_AUTO || d->schedule > DIT_SCHED_DYNAMIC)
    return fail(DIT_ERR_INVALID, "schedule=%d is not a dit_schedule", d->schedule);
  // the split schedule covers plain (one-segment, online-softmax) calls with
  // at least two key tiles, only when BALANCED asks for it.
  // AUTO never takes the split: on MI355X it measured slower on every shape
  // tried (Wan 480p: 130 against 109 us per kernel). The split kernel's loop
  // over pieces costs it spilled registers, and its key loop runs 56.5
  // cycles per MFMA against 43.6 in the one-workgroup-per-q-tile kernel.
  // Even with its loop at the per-q-tile rate it would gain little: the chip
  // is power-limited, and with every CU busy at full MFMA rate the clock
  // falls from about 2.1 GHz (the Wan 480p shard's 190 q-tiles) to about
  // 1.7 GHz, so 256 CUs deliver only about 9% more than 190, before each
  // piece's partial store and each q-tile's merge.
  if (d->schedule == DIT_SCHED_BALANCED && nq > 0 && nk >= 2 && d->kv_seg_len == 0 && !fm) {
    const int cus = device_cus();
    if (cus <= 0) return fail(DIT_ERR_HIP, "cannot query the compute-unit count of the current device");
    const SplitPlan sp = split_plan(nq, nk, cus);
    p.sk_grid = sp.grid;
    p.sk_main = sp.main;
    p.sk_kc = sp.kc;
  }
  // dynamic placement: every call without key segments. AUTO takes it from
  // kDynMinWaves waves of q-tiles: Wan 720p (2960 q-tiles, 11.6 waves)
  // measured 23.6-23.8 against 24.3-24.5 ms per kernel, while FLUX (432,
  // 1.7 waves) lost 11% (its second wave starts at once, and the contended
  // counters delay it more than the few tiles to rebalance save). The spare
  // workgroups are about what the fastest XCDs can take over (the XCDs'
  // clocks differ by about 5%).
  if ((d->schedule == DIT_SCHED_DYNAMIC || d->schedule == DIT_SCHED_AUTO) && nq > 0 && d->kv_seg_len == 0) {
    const int cus = device_cus();
    if (cus <= 0 && d->schedule == DIT_SCHED_DYNAMIC)
      return fail(DIT_ERR_HIP, "cannot query the compute-unit count of the current device");
    if (cus > 0 && (d->schedule == DIT_SCHED_DYNAMIC || nq >= kDynMinWaves * (int64_t)cus)) {
      const int64_t spare = nq / 16 > 8 ? nq / 16 : 8;
      if (nq + spare > INT32_MAX) return fail(DIT_ERR_UNSUPPORTED, "too many query tiles for one launch");
      p.dyn_grid = (int)(nq + spare);
      p.dyn_static = p.dyn_grid < cus ? p.dyn_grid : cus;
    }
  }
  size_t off = p.k_bytes + p.q_bytes;
  if (p.sk_grid > 0) {
    const size_t slots = 2 * (size_t)p.sk_grid;
    p.part_o_off = off;
    off += round_up(slots * kThreads * (d->d / 2) * sizeof(float), 256);
    p.part_l_off = off;
    off += round_up(slots * kBlockM * sizeof(float), 256);
    p.count_off = off;
    p.n_counts = nq;
    off += round_up((size_t)nq * sizeof(int32_t), 256);
  }
  if (p.dyn_grid > 0) {   // eight queue counters and the taken counter
    p.count_off = off;
    p.n_counts = 9;
    off += 256;
  }
  if (fm && d->kv_valid > 0 && d->s_q > 0) {
    const size_t bh = (size_t)d->B * d->H;
    const int64_t nqt = (d->s_q + kBlockM - 1) / kBlockM;
    p.fm = true;
    p.n_chunks = (d->s_kv + dit::kStatRows - 1) / dit::kStatRows;
    p.n_real = d->kv_seg_len > 0 ? (d->s_kv / d->kv_seg_len) * d->kv_valid : d->kv_valid;
    p.fm_part_off = off;
    off += round_up(bh * p.n_chunks * d->d * sizeof(float), 256);
    p.fm_kbar_off = off;
    off += round_up(bh * d->d * sizeof(float), 256);
    p.fm_r2_off = off;
    off += round_up(bh * p.n_chunks * sizeof(float), 256);
    p.fm_m_off = off;
    off += round_up(bh * (size_t)d->s_q * sizeof(float), 256);
    p.fm_ok_off = off;
    off += round_up(bh * (size_t)nqt * sizeof(int32_t), 256);
  }
  p.total = off;
  *pl = p;
  return DIT_OK;
}
// Device address of `scratch` on the current device, resolved once per
// device (with that device current) and cached; NULL with the status in rc
// when it cannot be resolved.
void *scratch_ptr(int *rc) {
  static std::atomic<void *> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *rc = fail(DIT_ERR_HIP, "no current HIP device (or device id beyond 63) for the static scratch");
    return nullptr;
  }
  void *ptr = cache[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *rc = fail(DIT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    cache[dev].store(ptr, std::memory_order_release);
  }
  *rc = DIT_OK;
  return ptr;
}
}  // namespace

extern "C" {

const char *dit_last_error(void) { return g_err; }

int dit_plan_padding(int s_valid, int multiple, int *s_pad_out) {
  if (s_pad_out == nullptr) return fail(DIT_ERR_INVALID, "s_pad_out is NULL");
  if (multiple <= 0 || s_valid < 0) return fail(DIT_ERR_INVALID, "need multiple > 0 and s_valid >= 0");
  const int64_t r = ((int64_t)s_valid + multiple - 1) / multiple * multiple;
  if (r > 0x7fffffffLL) return fail(DIT_ERR_INVALID, "padded length overflows int");
  *s_pad_out = (int)r;
  return ok();
}

int dit_attn_workspace_size(const dit_attn_desc *desc, size_t *bytes) {
  if (bytes == nullptr) return fail(DIT_ERR_INVALID, "bytes is NULL");
  float scale;
  int rc = validate_attn(desc, &scale);
  if (rc != DIT_OK) return rc;
  AttnPlan pl;
  if ((rc = plan_attn(desc, &pl)) != DIT_OK) return rc;
  *bytes = pl.total;
  return ok();
}

int dit_attn_fwd_noalloc(const dit_attn_desc *desc, void *stream) {
  float scale;
  int rc = validate_attn(desc, &scale);
  if (rc != DIT_OK) return rc;
  AttnPlan pl;
  if ((rc = plan_attn(desc, &pl)) != DIT_OK) return rc;
  if (pl.total > (size_t)DIT_NOALLOC_SCRATCH_BYTES)
    return fail(DIT_ERR_UNSUPPORTED, "this call needs %zu bytes of workspace; the static scratch of "
                "dit_attn_fwd_noalloc holds %zu (use dit_attn_fwd with a caller workspace)",
                pl.total, (size_t)DIT_NOALLOC_SCRATCH_BYTES);
  dit_attn_desc d = *desc;
  d.workspace = nullptr;
  d.workspace_bytes = 0;
  d.ws_counters_zero = 0;   // the array keeps whatever the last call left: clear the counters
  if (pl.total > 0) {
    d.workspace = scratch_ptr(&rc);
    if (rc != DIT_OK) return rc;
    d.workspace_bytes = DIT_NOALLOC_SCRATCH_BYTES;
  }
  return dit_attn_fwd(&d, stream);
}

int dit_attn_fwd(const dit_attn_desc *desc, void *stream) {
  float scale;
  int rc = validate_attn(desc, &scale);
  if (rc != DIT_OK) return rc;
  const dit_attn_desc &d = *desc;
  AttnPlan pl;
  if ((rc = plan_attn(desc, &pl)) != DIT_OK) return rc;
  const size_t need = pl.total;
  if (need > 0) {
    if (d.workspace == nullptr || d.workspace_bytes < need)
      return fail(DIT_ERR_INVALID, "workspace of %zu bytes required (got %zu)", need,
                  d.workspace == nullptr ? (size_t)0 : d.workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(d.workspace) & 255u) != 0) return fail(DIT_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  if (d.s_q == 0) return ok();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  dit::AttnParams p{};
  int64_t s3[3];
  resolve_strides(d.q_stride, d.H, d.s_q, d.d, s3);
  p.qs_b = s3[0]; p.qs_h = s3[1]; p.qs_s = s3[2];
  resolve_strides(d.k_stride, d.H, d.s_kv, d.d, s3);
  p.ks_b = s3[0]; p.ks_h = s3[1]; p.ks_s = s3[2];
  resolve_strides(d.v_stride, d.H, d.s_kv, d.d, s3);
  p.vs_b = s3[0]; p.vs_h = s3[1]; p.vs_s = s3[2];
  resolve_strides(d.o_stride, d.H, d.s_q, d.d, s3);
  p.os_b = s3[0]; p.os_h = s3[1]; p.os_s = s3[2];
  p.q = static_cast<const dit::bf16_t *>(d.q);
  p.k = static_cast<const dit::bf16_t *>(d.k);
  p.v = static_cast<const dit::bf16_t *>(d.v);
  p.o = d.o;
  p.lse = d.lse;
  p.B = d.B; p.H = d.H; p.s_q = d.s_q; p.s_kv = d.s_kv;
  p.q_valid = d.q_valid; p.kv_valid = d.kv_valid;
  p.q_seg_len = d.q_seg_len;
  p.kv_seg_len = d.kv_seg_len;
  p.n_kv_seg = d.kv_seg_len > 0 ? d.s_kv / d.kv_seg_len : 1;
  p.o_f32 = d.o_dtype == DIT_F32;
  p.n_qtiles = (d.s_q + dit::kAttnBlockM - 1) / dit::kAttnBlockM;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.sk_grid = pl.sk_grid;
  p.sk_main = pl.sk_main;
  p.sk_kc = pl.sk_kc;
  p.dyn_grid = pl.dyn_grid;
  p.dyn_static = pl.dyn_static;
  if (pl.sk_grid > 0) {
    char *ws = static_cast<char *>(d.workspace);
    p.sk_part_o = reinterpret_cast<float *>(ws + pl.part_o_off);
    p.sk_part_l = reinterpret_cast<float *>(ws + pl.part_l_off);
  }
  if (pl.n_counts > 0) p.sk_count = reinterpret_cast<int32_t *>(static_cast<char *>(d.workspace) + pl.count_off);

  // one pre-pass normalises and / or rotates K (valid rows) and Q (all rows)
  // into the workspace, and clears the schedule's counters
  const bool prepass = pl.k_bytes + pl.q_bytes > 0;
  if (prepass) {
    dit::RopeRotateParams r{};
    char *ws = static_cast<char *>(d.workspace);
    r.B = d.B; r.H = d.H; r.d = d.d;
    r.eps = d.norm_eps;
    if (!d.ws_counters_zero) {
      r.zero = p.sk_count;
      r.n_zero = (int32_t)pl.n_counts;
    }
    if (pl.k_bytes > 0) {
      dit::RopeSeg &g = r.seg[r.n_seg++];
      g.x = p.k; g.y = reinterpret_cast<dit::bf16_t *>(ws);
      g.cos_t = d.cos_k; g.sin_t = d.sin_k; g.norm_w = d.k_norm_w;
      g.xs_b = p.ks_b; g.xs_h = p.ks_h; g.xs_s = p.ks_s;
      g.S = d.s_kv; g.rows = d.kv_seg_len > 0 ? d.s_kv : d.kv_valid;   // segments: every segment's real rows
      p.k = g.y;
      p.ks_b = (int64_t)d.H * d.s_kv * d.d; p.ks_h = (int64_t)d.s_kv * d.d; p.ks_s = d.d;
    }
    if (pl.q_bytes > 0) {
      dit::RopeSeg &g = r.seg[r.n_seg++];
      g.x = p.q; g.y = reinterpret_cast<dit::bf16_t *>(ws + pl.k_bytes);
      g.cos_t = d.cos_q; g.sin_t = d.sin_q; g.norm_w = d.q_norm_w;
      g.xs_b = p.qs_b; g.xs_h = p.qs_h; g.xs_s = p.qs_s;
      g.S = d.s_q; g.rows = d.s_q;
      p.q = g.y;
      p.qs_b = (int64_t)d.H * d.s_q * d.d; p.qs_h = (int64_t)d.s_q * d.d; p.qs_s = d.d;
    }
    rc = hip_status(dit::launch_rope_rotate(r, st), "rotation launch");
    if (rc != DIT_OK) return rc;
  }
  if (pl.fm) {
    char *ws = static_cast<char *>(d.workspace);
    dit::FixedMParams f{};
    f.q = p.q; f.k = p.k;
    f.qs_b = p.qs_b; f.qs_h = p.qs_h; f.qs_s = p.qs_s;
    f.ks_b = p.ks_b; f.ks_h = p.ks_h; f.ks_s = p.ks_s;
    f.B = d.B; f.H = d.H; f.d = d.d; f.s_q = d.s_q; f.s_kv = d.s_kv;
    f.q_valid = d.q_valid; f.kv_valid = d.kv_valid; f.q_seg_len = d.q_seg_len; f.kv_seg_len = d.kv_seg_len;
    f.n_chunks = pl.n_chunks; f.n_real = pl.n_real; f.n_qtiles = p.n_qtiles;
    f.c2 = p.scale_log2;
    f.part = reinterpret_cast<float *>(ws + pl.fm_part_off);
    f.kbar = reinterpret_cast<float *>(ws + pl.fm_kbar_off);
    f.r2 = reinterpret_cast<float *>(ws + pl.fm_r2_off);
    f.m = reinterpret_cast<float *>(ws + pl.fm_m_off);
    f.ok = reinterpret_cast<int32_t *>(ws + pl.fm_ok_off);
    rc = hip_status(dit::launch_fixed_m(f, st), "fixed-m statistics launch");
    if (rc != DIT_OK) return rc;
    p.fm_m = f.m;
    p.fm_ok = f.ok;
  }
  if (pl.n_counts > 0 && !prepass && !d.ws_counters_zero) {
    // schedule counters start at zero (a fill kernel, not a memset node)
    rc = hip_status(dit::launch_zero_i32(p.sk_count, pl.n_counts, st), "counter clear launch");
    if (rc != DIT_OK) return rc;
  }
  return hip_status(dit::launch_attn_fwd(p, d.d, st), "attention launch");
}

int dit_lse_merge(int n_parts, const void *const *o_parts, const float *const *lse_parts, int part_dtype, int B,
                  int H, int S, int d, int q_valid, void *o_out, int out_dtype, float *lse_out, void *stream) {
  if (n_parts < 1 || n_parts > dit::kMaxMergeParts)
    return fail(DIT_ERR_INVALID, "n_parts=%d must lie in [1, %d]", n_parts, dit::kMaxMergeParts);
  if (o_parts == nullptr || lse_parts == nullptr) return fail(DIT_ERR_INVALID, "o_parts and lse_parts must be non-NULL host arrays");
  if (B < 1 || H < 1 || S < 0) return fail(DIT_ERR_INVALID, "need B >= 1, H >= 1, S >= 0");
  if (d <= 0 || d % 2) return fail(DIT_ERR_INVALID, "d=%d must be positive and even", d);
  if (d != 64 && d != 128) return fail(DIT_ERR_UNSUPPORTED, "merge kernels exist for d in {64, 128}");
  if (q_valid < 0 || q_valid > S) return fail(DIT_ERR_INVALID, "q_valid=%d must lie in [0, S=%d]", q_valid, S);
  if ((part_dtype != DIT_BF16 && part_dtype != DIT_F32) || (out_dtype != DIT_BF16 && out_dtype != DIT_F32))
    return fail(DIT_ERR_INVALID, "dtypes must be DIT_BF16 or DIT_F32");
  if (S > 0 && o_out == nullptr) return fail(DIT_ERR_INVALID, "o_out is NULL");
  for (int k = 0; k < n_parts; ++k) {
    if (S > 0 && (o_parts[k] == nullptr || lse_parts[k] == nullptr))
      return fail(DIT_ERR_INVALID, "part %d has a NULL pointer", k);
    if ((reinterpret_cast<uintptr_t>(o_parts[k]) & 3u) || (reinterpret_cast<uintptr_t>(lse_parts[k]) & 3u))
      return fail(DIT_ERR_UNSUPPORTED, "part %d pointers must be 4-byte aligned", k);
  }
  if (reinterpret_cast<uintptr_t>(o_out) & 3u) return fail(DIT_ERR_UNSUPPORTED, "o_out must be 4-byte aligned");
  const int64_t rows = (int64_t)B * H * S;
  if (rows > 0x7fffffffLL) return fail(DIT_ERR_UNSUPPORTED, "too many rows");
  if (rows == 0) return ok();
  dit::MergeParams p{};
  for (int k = 0; k < n_parts; ++k) {
    p.o_parts[k] = o_parts[k];
    p.lse_parts[k] = lse_parts[k];
  }
  p.o_out = o_out;
  p.lse_out = lse_out;
  p.n_parts = n_parts;
  p.part_f32 = part_dtype == DIT_F32;
  p.out_f32 = out_dtype == DIT_F32;
  p.rows = (int32_t)rows;
  p.S = S;
  p.d = d;
  p.q_valid = q_valid;
  return hip_status(dit::launch_lse_merge(p, reinterpret_cast<hipStream_t>(stream)), "merge launch");
}

int dit_rope_split_tables(const int32_t *pos, int S, int n_axes, const int32_t *axis_channels, int d, float theta,
                          float *cos_out, float *sin_out, void *stream) {
  if (S < 0) return fail(DIT_ERR_INVALID, "S must be >= 0");
  if (n_axes < 1 || n_axes > 8) return fail(DIT_ERR_INVALID, "n_axes=%d must lie in [1, 8]", n_axes);
  if (axis_channels == nullptr) return fail(DIT_ERR_INVALID, "axis_channels is NULL");
  if (d < 2 || d > 2 * dit::kMaxPairs || d % 2) return fail(DIT_ERR_INVALID, "d=%d must be even and in [2, %d]", d, 2 * dit::kMaxPairs);
  if (!(theta > 0.0f) || !std::isfinite(theta)) return fail(DIT_ERR_INVALID, "theta must be finite and positive");
  if ((int64_t)S * (d / 2) > 0x7fffffffLL) return fail(DIT_ERR_UNSUPPORTED, "S * d/2 must be below 2^31");
  int sum = 0;
  for (int a = 0; a < n_axes; ++a) {
    if (axis_channels[a] <= 0 || axis_channels[a] % 2 || axis_channels[a] > d)
      return fail(DIT_ERR_INVALID, "axis %d has %d channels: each axis needs a positive even count <= d", a,
                  axis_channels[a]);
    sum += axis_channels[a];
  }
  if (sum != d) return fail(DIT_ERR_INVALID, "axis channels sum to %d, not d=%d", sum, d);
  if (S > 0 && (pos == nullptr || cos_out == nullptr || sin_out == nullptr))
    return fail(DIT_ERR_INVALID, "pos, cos_out and sin_out must be non-NULL");
  if (S == 0) return ok();
  dit::TableParams p{};
  int j = 0;
  for (int a = 0; a < n_axes; ++a) {
    const int c = axis_channels[a];
    for (int k = 0; k < c / 2; ++k, ++j) {
      p.freq[j] = std::pow((double)theta, -2.0 * k / (double)c);
      p.axis[j] = (uint8_t)a;
    }
  }
  p.pos = pos;
  p.cos_out = cos_out;
  p.sin_out = sin_out;
  p.S = S;
  p.n_axes = n_axes;
  p.half_d = d / 2;
  return hip_status(dit::launch_rope_tables(p, reinterpret_cast<hipStream_t>(stream)), "table launch");
}

int dit_pad_tokens(const void *in, void *out, int B, int s_valid, int s_pad, int64_t row_bytes, void *stream) {
  if (B < 1 || s_valid < 0 || s_pad < s_valid || row_bytes <= 0)
    return fail(DIT_ERR_INVALID, "need B >= 1, 0 <= s_valid <= s_pad, row_bytes > 0");
  if (s_pad > 0 && out == nullptr) return fail(DIT_ERR_INVALID, "out is NULL");
  if (s_valid > 0 && in == nullptr) return fail(DIT_ERR_INVALID, "in is NULL");
  if (in != nullptr && in == out) return fail(DIT_ERR_INVALID, "in and out must not alias");
  if (B > 65535) return fail(DIT_ERR_UNSUPPORTED, "B > 65535 (one grid row per batch)");
  return hip_status(dit::launch_row_copy(in, out, B, s_valid, s_pad, s_valid, row_bytes, reinterpret_cast<hipStream_t>(stream)),
                    "pad launch");
}

int dit_pad_tokens_rope(const void *in, void *out, int B, int s_valid, int s_pad, int T, int H, int d, int n_rot,
                        const float *cos_t, const float *sin_t, void *stream) {
  if (B < 1 || s_valid < 0 || s_pad < s_valid || T < 1 || H < 1 || n_rot < 0 || n_rot > T)
    return fail(DIT_ERR_INVALID, "need B >= 1, 0 <= s_valid <= s_pad, T >= 1, H >= 1, 0 <= n_rot <= T");
  if (d != 64 && d != 128) return fail(DIT_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (s_pad > 0 && out == nullptr) return fail(DIT_ERR_INVALID, "out is NULL");
  if (s_valid > 0 && in == nullptr) return fail(DIT_ERR_INVALID, "in is NULL");
  if (s_valid > 0 && n_rot > 0 && (cos_t == nullptr || sin_t == nullptr))
    return fail(DIT_ERR_INVALID, "cos_t / sin_t are NULL with n_rot > 0");
  if (in != nullptr && in == out) return fail(DIT_ERR_INVALID, "in and out must not alias");
  const uintptr_t al = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out) |
                       reinterpret_cast<uintptr_t>(cos_t) | reinterpret_cast<uintptr_t>(sin_t);
  if (al % 16 != 0) return fail(DIT_ERR_INVALID, "in, out, cos_t and sin_t must be 16-byte aligned");
  if (B > 65535) return fail(DIT_ERR_UNSUPPORTED, "B > 65535 (one grid row per batch)");
  if ((int64_t)T * H * (d / 16) * s_pad >= (int64_t(1) << 31))
    return fail(DIT_ERR_UNSUPPORTED, "T * H * d/16 * s_pad must be below 2^31");
  dit::PadRopeParams p{};
  p.in = static_cast<const dit::bf16_t *>(in);
  p.out = static_cast<dit::bf16_t *>(out);
  p.cos_t = cos_t;
  p.sin_t = sin_t;
  p.s_valid = s_valid;
  p.s_pad = s_pad;
  p.T = T;
  p.H = H;
  p.n_rot = n_rot;
  return hip_status(dit::launch_pad_rope(p, B, d, reinterpret_cast<hipStream_t>(stream)), "pad+rope launch");
}

int dit_unpad_tokens(const void *in, void *out, int B, int s_pad, int s_valid, int64_t row_bytes, void *stream) {
  if (B < 1 || s_valid < 0 || s_pad < s_valid || row_bytes <= 0)
    return fail(DIT_ERR_INVALID, "need B >= 1, 0 <= s_valid <= s_pad, row_bytes > 0");
  if (s_valid > 0 && (out == nullptr || in == nullptr)) return fail(DIT_ERR_INVALID, "in and out must be non-NULL");
  if (in != nullptr && in == out) return fail(DIT_ERR_INVALID, "in and out must not alias (no in-place unpad)");
  if (B > 65535) return fail(DIT_ERR_UNSUPPORTED, "B > 65535 (one grid row per batch)");
  return hip_status(dit::launch_row_copy(in, out, B, s_pad, s_valid, s_valid, row_bytes, reinterpret_cast<hipStream_t>(stream)),
                    "unpad launch");
}

}  // extern "C"
