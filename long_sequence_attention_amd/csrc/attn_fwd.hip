// Attention forward for gfx950: bf16 MFMA (v_mfma_f32_32x32x16_bf16) with
// fp32 accumulation, online softmax in exp2 form, exact tail-pad masking,
// split-halves RoPE fused into the Q load, and a K rotation pre-pass.
//
// What is computed (the pages' problem statement): for each (b, h) and query
// row i < q_valid, O_i = sum_{j < kv_valid} softmax_j(scale * q'_i . k'_j) v_j
// and LSE_i = ln sum_j exp(scale * q'_i . k'_j), with q', k' the split-halves
// rotations (Difflet PR #153, FLUX split-RoPE and Wan padding commits; mstar
// PR #376 for the natural-log LSE returned beside O; maxdiffusion PR #491 for
// masking pads through the real KV length).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//   * Each wave owns 32 query rows and computes S^T = K Q^T, so a lane holds
//     16 scores of ONE query (lane % 32) per 32-key block: the row max is an
//     in-register reduction plus one v_permlane32_swap with lane ^ 32.
//   * Q stays in registers (bf16, rotated once) as the B operand of S^T.
//   * K and V tiles (64 keys x d) move HBM -> LDS with buffer loads that
//     write LDS directly (no VGPR staging). Each load's buffer view ends at
//     row kv_valid, so tail pads and rows past the tensor arrive as zeros:
//     no pad byte, NaN or Inf ever reaches LDS.
//   * Both tiles are row-major in LDS with the 16-byte chunks of a row
//     permuted by an XOR of the row index, so the K operand reads (16 rows,
//     one chunk) and the V operand reads hit distinct banks.
//   * The V^T operand of O^T = V^T P^T is produced by LDS transpose reads
//     (ds_read_b64_tr_b16) from the row-major V tile.
//   * The key order inside a 32-key block is permuted when K rows are read
//     (MFMA row m = 16a+8b+4c+j holds key 16a+8c+4b+j) so the scores a lane
//     gets back from the S^T MFMA are exactly the 8-key runs it feeds as the
//     P^T operand: P goes from accumulator to operand with one bf16 pack.
//   * Software pipeline: K runs one tile ahead of V. While the softmax of
//     tile t runs on the VALU, the S MFMAs of tile t+1 run on the matrix
//     cores (interleaved with sched_group_barrier); then P(t).V(t) runs while
//     the row max of tile t+1 is taken. Two tiles per loop iteration keep
//     the score registers and LDS buffer parity static.
//   * exp2 with scale*log2(e) folded into one FMA, and a lazy rescale: the
//     running max is only raised (and O, l rescaled) when a tile max exceeds
//     it by more than 8 (log2 units), so p <= 2^8 stays exact in fp32/bf16
//     range. The result is unchanged in exact arithmetic.
//   * Pad keys: tiles past kv_valid are never visited; in the tail tile,
//     scores of keys >= kv_valid are replaced by -inf with a select.
//   * Pad query rows are computed but overwritten by a select in the epilogue.
//   * XCD-aware workgroup order: consecutive q-tiles of a head run on one
//     XCD so its K/V stay in that XCD's L2.
#include "common.h"

namespace dit {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup
constexpr float kLazyRescale = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

__device__ __forceinline__ u32x4 ldg16(const bf16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ void rotate8(u32x4 &lo, u32x4 &hi, const float *c, const float *s) {
  const float4 c0 = *reinterpret_cast<const float4 *>(c);
  const float4 c1 = *reinterpret_cast<const float4 *>(c + 4);
  const float4 s0 = *reinterpret_cast<const float4 *>(s);
  const float4 s1 = *reinterpret_cast<const float4 *>(s + 4);
  const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  u32x4 nlo, nhi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x1a = bf16_lo(lo[w]), x1b = bf16_hi(lo[w]);
    const float x2a = bf16_lo(hi[w]), x2b = bf16_hi(hi[w]);
    const float ca = cv[2 * w], cb = cv[2 * w + 1], sa = sv[2 * w], sb = sv[2 * w + 1];
    const float y1a = fmaf(x1a, ca, -x2a * sa), y1b = fmaf(x1b, cb, -x2b * sb);
    const float y2a = fmaf(x2a, ca, x1a * sa), y2b = fmaf(x2b, cb, x1b * sb);
    nlo[w] = pack_bf16x2(y1a, y1b);
    nhi[w] = pack_bf16x2(y2a, y2b);
  }
  lo = nlo;
  hi = nhi;
}

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;
  static constexpr int RPB = 16 / CPR;
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / 4;
  static constexpr int K0 = 0, V0 = 2 * TILE_BYTES;
  __device__ static constexpr int fk(int r) { return (r / RPB) % CPR; }
  __device__ static constexpr int fv(int r) { return 4 * ((r / RPB) % (4 / RPB)); }
};

// Issue this wave's share of tile t of K or V as buffer->LDS loads. The
// buffer view starts at the tile's first row and ends at row kv_valid, so
// rows past kv_valid (tail pads, or past the tensor) arrive as zeros. The
// view is rebuilt per tile with scalar arithmetic: the hardware range check
// covers the per-lane offset, not a scalar offset.
template <int D>
__device__ __forceinline__ void issue_rows(char *dst, const bf16_t *base, int row_bytes, int t, int kv_valid,
                                           const int *off, int wave) {
  using G = Geo<D>;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(base)) + (int64_t)t * BN * row_bytes, 0,
      (kv_valid - t * BN) * row_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < G::LOADS_PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + (wave * G::LOADS_PER_WAVE + i) * 1024), 16,
                                             off[i], 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void qk_tile(const char *kt, const int *kaddr, const bf16x8 *qop, f32x16 *sacc) {
  constexpr int DK = D / 16;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    sacc[blk] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kt + blk * 32 * D * 2 + kaddr[dk]);
      sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[dk], sacc[blk], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void mask_tail(f32x16 *sacc, int j0, int kv_valid, int hf) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + blk * 32 + ((r & 8) << 1) + 8 * hf + (r & 7);
      sacc[blk][r] = (key < kv_valid) ? sacc[blk][r] : -INFINITY;
    }
  }
}

__device__ __forceinline__ float pair_max(const f32x16 *s) {
  float m0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
  float m1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) {
    m0 = fmaxf(fmaxf(m0, s[0][r]), s[0][r + 1]);
    m1 = fmaxf(fmaxf(m1, s[1][r]), s[1][r + 1]);
  }
  float m = fmaxf(fmaxf(m0, s[0][15]), fmaxf(m1, s[1][15]));
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

template <int D>
struct StepCtx {
  char *smem;
  const bf16_t *kbase, *vbase;
  const int *koff, *voff, *kaddr, *vaddr;
  const bf16x8 *qop;
  int ks_bytes, vs_bytes, kv_valid, n_tiles, wave, hf;
  float c2;
};

template <int D, bool HAS_NEXT, bool MASK_NEXT>
__device__ __forceinline__ void step(const StepCtx<D> &cx, int t, int par, const f32x16 *scur, f32x16 *snext,
                                     f32x16 *acc_o, float &m_run, float &l_run) {
  using G = Geo<D>;
  constexpr int DK = D / 16, DB = D / 32;
  if (t + 2 < cx.n_tiles)
    issue_rows<D>(cx.smem + G::K0 + par * G::TILE_BYTES, cx.kbase, cx.ks_bytes, t + 2, cx.kv_valid, cx.koff, cx.wave);
  if (HAS_NEXT)
    issue_rows<D>(cx.smem + G::V0 + (par ^ 1) * G::TILE_BYTES, cx.vbase, cx.vs_bytes, t + 1, cx.kv_valid, cx.voff, cx.wave);
  const char *vt = cx.smem + G::V0 + par * G::TILE_BYTES;

  const float neg_m = -m_run;
  bf16x8 pop[2][2];
  float ps0 = 0.f, ps1 = 0.f;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      f32x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(scur[blk][8 * a + e], cx.c2, neg_m));
      pop[blk][a] = __builtin_convertvector(pv, bf16x8);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        ps0 += pv[e];
        ps1 += pv[e + 1];
      }
    }
  }
  if (HAS_NEXT) {
    qk_tile<D>(cx.smem + G::K0 + (par ^ 1) * G::TILE_BYTES, cx.kaddr, cx.qop, snext);
    if (MASK_NEXT) mask_tail(snext, (t + 1) * BN, cx.kv_valid, cx.hf);
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const char *src = vt + (blk * 32 + a * 16) * D * 2 + cx.vaddr[db];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(src));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(src + 4 * D * 2));
        const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pop[blk][a], acc_o[db], 0, 0, 0);
      }
    }
  }
  float mts = 0.f;
  if (HAS_NEXT) mts = pair_max(snext) * cx.c2;
  if (HAS_NEXT && !MASK_NEXT) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * DK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 96 / (2 * DK), 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
  }
  l_run += ps0 + ps1;

  if (HAS_NEXT) {
    const bool upd = mts > m_run + kLazyRescale;
    if (__any(upd)) {
      const float m_new = upd ? mts : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnParams p) {
  using G = Geo<D>;
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = G::CPR;
  __shared__ __attribute__((aligned(1024))) char smem[4 * G::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int h = bh % p.H;
  const int b = bh / p.H;

  const bf16_t *qbase = p.q + b * p.qs_b + h * p.qs_h;
  const bf16_t *kbase = p.k + b * p.ks_b + h * p.ks_h;
  const bf16_t *vbase = p.v + b * p.vs_b + h * p.vs_h;
  const int kv_valid = p.kv_valid;
  const int n_tiles = (kv_valid + BN - 1) / BN;

  const int ks_bytes = (int)(p.ks_s * 2), vs_bytes = (int)(p.vs_s * 2);

  int koff[G::LOADS_PER_WAVE], voff[G::LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < G::LOADS_PER_WAVE; ++i) {
    const int s = (wave * G::LOADS_PER_WAVE + i) * 64 + lane;
    const int r = s / CPR, pos = s % CPR;
    koff[i] = r * ks_bytes + ((pos ^ G::fk(r)) * 16);
    voff[i] = r * vs_bytes + ((pos ^ G::fv(r)) * 16);
  }
  if (n_tiles > 0) {
    issue_rows<D>(smem + G::K0, kbase, ks_bytes, 0, kv_valid, koff, wave);
    issue_rows<D>(smem + G::V0, vbase, vs_bytes, 0, kv_valid, voff, wave);
  }
  if (n_tiles > 1) issue_rows<D>(smem + G::K0 + G::TILE_BYTES, kbase, ks_bytes, 1, kv_valid, koff, wave);

  const int qrow = qt * BM + wave * 32 + l32;
  bf16x8 qop[DK];
  {
    u32x4 raw[DK];
    const bool in_q = qrow < p.s_q;
    const bf16_t *qr = qbase + (int64_t)(in_q ? qrow : 0) * p.qs_s;
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) raw[dk] = in_q ? ldg16(qr + dk * 16 + hf * 8) : u32x4{0u, 0u, 0u, 0u};
    if (p.cos_q != nullptr) {
      const int64_t trow = (int64_t)(in_q ? qrow : 0) * (D / 2);
#pragma unroll
      for (int dk = 0; dk < DK / 2; ++dk) {
        const int i0 = dk * 16 + hf * 8;
        rotate8(raw[dk], raw[dk + DK / 2], p.cos_q + trow + i0, p.sin_q + trow + i0);
      }
    }
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) qop[dk] = __builtin_bit_cast(bf16x8, raw[dk]);
  }

  const int kperm = (l32 & 16) + ((l32 & 4) << 1) + ((l32 & 8) >> 1) + (l32 & 3);
  int kaddr[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk)
    kaddr[dk] = kperm * (D * 2) + (((2 * dk + hf) ^ G::fk(kperm)) * 16);
  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
  const int vrow = 8 * (tg >> 1) + te;
  int vaddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 4 * db + 2 * (tg & 1) + (tq >> 1);
    vaddr[db] = vrow * (D * 2) + ((chunk ^ G::fv(vrow)) * 16) + 8 * (tq & 1);
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};

  const float c2 = p.scale_log2;
  f32x16 sa[2], sb[2];
  if (n_tiles > 0) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    qk_tile<D>(smem + G::K0, kaddr, qop, sa);
    __syncthreads();
    if (BN > kv_valid) mask_tail(sa, 0, kv_valid, hf);
    m_run = pair_max(sa) * c2;
  }
  StepCtx<D> cx{smem, kbase, vbase, koff, voff, kaddr, vaddr, qop, ks_bytes, vs_bytes, kv_valid, n_tiles, wave, hf, c2};
  // steady state: tiles t, t+1, t+2 all full; two tiles per iteration so the
  // score registers alternate roles and the LDS buffer parity is static
  int t = 0;
  for (; t + 3 < n_tiles; t += 2) {
    step<D, true, false>(cx, t, 0, sa, sb, acc_o, m_run, l_run);
    step<D, true, false>(cx, t + 1, 1, sb, sa, acc_o, m_run, l_run);
  }
  // at most three tiles remain (t is even here): tile t+1 may be the masked tail
  if (t + 1 < n_tiles) {
    if ((t + 2) * BN > kv_valid) step<D, true, true>(cx, t, 0, sa, sb, acc_o, m_run, l_run);
    else step<D, true, false>(cx, t, 0, sa, sb, acc_o, m_run, l_run);
    ++t;
    if (t + 1 < n_tiles) {
      if ((t + 2) * BN > kv_valid) step<D, true, true>(cx, t, 1, sb, sa, acc_o, m_run, l_run);
      else step<D, true, false>(cx, t, 1, sb, sa, acc_o, m_run, l_run);
      ++t;
      step<D, false, false>(cx, t, 0, sa, sb, acc_o, m_run, l_run);
    } else {
      step<D, false, false>(cx, t, 1, sb, sa, acc_o, m_run, l_run);
    }
  } else if (t < n_tiles) {
    step<D, false, false>(cx, t, 0, sa, sb, acc_o, m_run, l_run);
  }

  // ---- epilogue: O = acc / l; LSE = (m + log2 l) ln 2; pad rows by select
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  if (qrow >= p.s_q) return;
  const bool row_ok = (qrow < p.q_valid) && (kv_valid > 0);
  const float inv = row_ok ? 1.0f / l_tot : 0.0f;
  const int64_t obase = b * p.os_b + h * p.os_h + (int64_t)qrow * p.os_s;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + 8 * i + 4 * hf;
      float o4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o4[j] = row_ok ? acc_o[db][4 * i + j] * inv : 0.0f;
      if (p.o_f32) {
        float *op = reinterpret_cast<float *>(p.o) + obase + d0;
        *reinterpret_cast<float4 *>(op) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      } else {
        bf16_t *op = reinterpret_cast<bf16_t *>(p.o) + obase + d0;
        *reinterpret_cast<u32x2 *>(op) = u32x2{pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
      }
    }
  }
  if (p.lse != nullptr && hf == 0) {
    const float lse = row_ok ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    p.lse[((int64_t)b * p.H + h) * p.s_q + qrow] = lse;
  }
}

__global__ __launch_bounds__(256) void rope_rotate_kernel(RopeRotateParams p) {
  const int runs = p.d / 16;
  const int half = p.d / 2;
  const int64_t total = (int64_t)p.B * p.H * p.valid * runs;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(t % runs);
    int64_t r = t / runs;
    const int s = (int)(r % p.valid);
    r /= p.valid;
    const int h = (int)(r % p.H);
    const int b = (int)(r / p.H);
    const bf16_t *xr = p.x + b * p.xs_b + h * p.xs_h + (int64_t)s * p.xs_s;
    bf16_t *yr = p.y + (((int64_t)b * p.H + h) * p.S + s) * p.d;
    u32x4 lo = ldg16(xr + c * 8);
    u32x4 hi = ldg16(xr + half + c * 8);
    const int64_t to = (int64_t)s * half + c * 8;
    rotate8(lo, hi, p.cos_t + to, p.sin_t + to);
    *reinterpret_cast<u32x4 *>(yr + c * 8) = lo;
    *reinterpret_cast<u32x4 *>(yr + half + c * 8) = hi;
  }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams &p, int d, hipStream_t stream) {
  const int64_t nblocks = (int64_t)p.n_qtiles * p.H * p.B;
  if (nblocks <= 0) return hipSuccess;
  if (d == 128) {
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3((unsigned)nblocks), dim3(NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3((unsigned)nblocks), dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_rope_rotate(const RopeRotateParams &p, hipStream_t stream) {
  const int64_t total = (int64_t)p.B * p.H * p.valid * (p.d / 16);
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_rotate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

int attn_block_m() { return BM; }

}  // namespace dit
