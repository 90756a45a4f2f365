// Attention forward for gfx950: bf16 MFMA (v_mfma_f32_32x32x16_bf16) with
// fp32 accumulation, online softmax in exp2 form, exact tail-pad masking,
// and a pre-pass that applies the optional per-head q/k RMS normalisation and
// the split-halves RoPE to Q and K once per call.
//
// What is computed (the pages' problem statement): for each (b, h) and query
// row i < q_valid, O_i = sum_{j < kv_valid} softmax_j(scale * q'_i . k'_j) v_j
// and LSE_i = ln sum_j exp(scale * q'_i . k'_j), with q', k' the split-halves
// rotations (Difflet PR #153, FLUX split-RoPE and Wan padding commits; mstar
// PR #376 for the natural-log LSE returned beside O; maxdiffusion PR #491 for
// masking pads through the real KV length).
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   * Each wave owns 32 query rows and computes S^T = K Q^T, so a lane holds
//     16 scores of ONE query (lane % 32) per 32-key block: the row max is an
//     in-register reduction plus one v_permlane32_swap with lane ^ 32.
//   * Q stays in registers (bf16, already rotated) as the B operand of S^T.
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
//   * Software pipeline: K runs one tile ahead of V. The softmax of tile t
//     (VALU) is interleaved (sched_group_barrier) with the S MFMAs of tile
//     t+1 and the P(t).V(t) MFMAs, split so both MFMA groups carry VALU
//     work; the row max of tile t+1 is taken beside P(t).V(t). Two tiles
//     per loop iteration keep the score registers and LDS buffer parity
//     static.
//   * exp2 with scale*log2(e) folded into one FMA, and a lazy rescale: the
//     running max is only raised (and O, l rescaled) when a tile max exceeds
//     it by more than 8 (log2 units), so p <= 2^8 stays exact in fp32/bf16
//     range. The result is unchanged in exact arithmetic.
//   * Pad keys: tiles past kv_valid are never visited; in the tail tile,
//     scores of keys >= kv_valid are replaced by -inf with a select.
//   * Pad query rows are computed but overwritten by a select in the
//     epilogue; a wave whose 32 rows are all tail pads skips the arithmetic
//     (it only issues its share of the K/V loads and meets the barriers),
//     which lowers the power drawn by the last q-tile of each head.
//   * XCD-aware workgroup order: consecutive q-tiles of a head run on one
//     XCD so its K/V stay in that XCD's L2.
//   * Segmented keys (ring layout): attn_fwd_seg_kernel runs the same key
//     pipeline once per segment's real tiles, carrying the softmax state.
//   * Fixed-m softmax (opt-in): a q-tile whose a-priori row bounds
//     (fixed_m.hip) are tight enough runs the FIXED instance of the step,
//     with the bound as its maximum: no running max and no rescale.
#include "common.h"

namespace dit {

namespace {

constexpr int BM = kAttnBlockM;   // query rows per workgroup
constexpr int BN = kAttnBlockN;   // keys per tile
constexpr int NT = kAttnThreads;   // threads per workgroup
constexpr float kLazyRescale = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

__device__ __forceinline__ u32x4 ldg16(const bf16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Race check build (compiled with -DDIT_DEBUG_SYNC=1 into a separate
// library): every wave waits for all of its outstanding global and LDS
// accesses and meets the others at a barrier after each DMA issue and each
// LDS read phase. The arithmetic is unchanged, so its results must equal
// the pipelined build's bit for bit; a missing wait or barrier in the
// pipeline would show up as a difference.
#ifndef DIT_DEBUG_SYNC
#define DIT_DEBUG_SYNC 0
#endif
// Clock probe build (compiled with -DDIT_CLOCK_PROBE=1 into a separate
// library): the first thread of each of the first kClockProbeWgs workgroups
// records the shader-clock counter (s_memtime) and the constant 100 MHz
// counter (s_memrealtime) when its key loop starts and when it ends (words
// 0-3 of its 8) and the loop's key-tile count (word 6); in the
// one-workgroup-per-q-tile kernel also the 100 MHz counter when the
// workgroup starts (word 4) and once every wave's O / LSE stores have
// completed (word 5). Under the split schedule the stamps are of the
// workgroup's last piece. Clock = loop cycles / loop time; the entry and
// exit stamps place the prologue, the epilogue and the time outside the
// workgroups in the launch. The arithmetic is unchanged.
#ifndef DIT_CLOCK_PROBE
#define DIT_CLOCK_PROBE 0
#endif
#if DIT_CLOCK_PROBE
constexpr int kClockProbeWgs = 4096;
__device__ unsigned long long g_clock_probe[kClockProbeWgs * 8];
#endif
__device__ __forceinline__ void clock_mark(int k) {
#if DIT_CLOCK_PROBE
  if (threadIdx.x == 0 && blockIdx.x < kClockProbeWgs) {
    g_clock_probe[blockIdx.x * 8 + 2 * k] = __builtin_amdgcn_s_memtime();
    g_clock_probe[blockIdx.x * 8 + 2 * k + 1] = __builtin_amdgcn_s_memrealtime();
  }
#else
  (void)k;
#endif
}
// the number of key tiles the stamped loop ran (word 6)
__device__ __forceinline__ void clock_note_tiles(int n) {
#if DIT_CLOCK_PROBE
  if (threadIdx.x == 0 && blockIdx.x < kClockProbeWgs) g_clock_probe[blockIdx.x * 8 + 6] = (unsigned long long)n;
#else
  (void)n;
#endif
}
// k = 0: workgroup entry; k = 1: after the workgroup's stores completed
__device__ __forceinline__ void clock_edge(int k) {
#if DIT_CLOCK_PROBE
  if (k == 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are done
    __syncthreads();
  }
  if (threadIdx.x == 0 && blockIdx.x < kClockProbeWgs)
    g_clock_probe[blockIdx.x * 8 + 4 + k] = __builtin_amdgcn_s_memrealtime();
#else
  (void)k;
#endif
}

__device__ __forceinline__ void debug_sync() {
  if constexpr (DIT_DEBUG_SYNC != 0) {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
    __syncthreads();
  }
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
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / kAttnWaves;
  static constexpr int K0 = 0, V0 = 2 * TILE_BYTES;
  __device__ static constexpr int fk(int r) { return (r / RPB) % CPR; }
  __device__ static constexpr int fv(int r) { return 4 * ((r / RPB) % (4 / RPB)); }
};

// One 16-byte-per-lane buffer load that writes LDS directly (lane l's 16
// bytes land at M0 + 16 l). Issued as inline assembly so the compiler does
// not treat it as a pending LDS write that every later LDS read must wait
// for: the kernel orders these loads itself (s_waitcnt vmcnt(0) and a
// barrier before a filled buffer is read). M0 = wbase + OFF is formed inside
// the statement (one wait state before the load reads it), so the 16
// distinct LDS targets of a step do not each hold an SGPR. M0 is a declared
// output of the statement ("={m0}"), so the compiler knows the statement
// overwrites it and keeps no value of its own there across it.
template <int OFF>
__device__ __forceinline__ void lds_dma16(uint32_t wbase, int voff, i32x4 rsrc) {
  uint32_t m0_out;
  asm volatile("s_add_u32 m0, %1, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               : "={m0}"(m0_out)
               : "s"(wbase), "v"(voff), "s"(rsrc), "i"(OFF)
               : "memory", "scc");
  (void)m0_out;
}

// Issue this wave's share of tile t of K or V into LDS buffer BUF (byte
// offset in the tile area) as buffer->LDS loads; wbase is the LDS address of
// this wave's first 1 KB slot. The buffer view starts at the tile's first
// row and ends at row kv_valid, so rows past kv_valid (tail pads, or past
// the tensor) arrive as zeros. The view is rebuilt per tile with scalar
// arithmetic: the hardware range check covers the per-lane offset, not a
// scalar offset.
template <int D, int BUF>
__device__ __forceinline__ void issue_rows(uint32_t wbase, const bf16_t *base, int row_bytes, int t, int kv_valid,
                                           const int *off) {
  using G = Geo<D>;
  const uint64_t addr = reinterpret_cast<uint64_t>(base) + (uint64_t)((int64_t)t * BN * row_bytes);
  // descriptor: base, stride 0, num_records = bytes to row kv_valid, raw buffer
  const i32x4 rs = {(int32_t)(uint32_t)addr, (int32_t)((addr >> 32) & 0xffffu), (kv_valid - t * BN) * row_bytes,
                    0x00020000};
  if constexpr (G::LOADS_PER_WAVE > 0) lds_dma16<BUF + 0 * 1024>(wbase, off[0], rs);
  if constexpr (G::LOADS_PER_WAVE > 1) lds_dma16<BUF + 1 * 1024>(wbase, off[1], rs);
  if constexpr (G::LOADS_PER_WAVE > 2) lds_dma16<BUF + 2 * 1024>(wbase, off[2], rs);
  if constexpr (G::LOADS_PER_WAVE > 3) lds_dma16<BUF + 3 * 1024>(wbase, off[3], rs);
  static_assert(G::LOADS_PER_WAVE <= 4, "at most four 1 KB loads per wave and tile");
}

// Runtime buffer parity -> compile-time LDS offset.
template <int D, int BUF0>
__device__ __forceinline__ void issue_rows_par(int par, uint32_t wbase, const bf16_t *base, int row_bytes, int t,
                                               int kv_valid, const int *off) {
  if (par) issue_rows<D, BUF0 + Geo<D>::TILE_BYTES>(wbase, base, row_bytes, t, kv_valid, off);
  else issue_rows<D, BUF0>(wbase, base, row_bytes, t, kv_valid, off);
}

// S^T of one key tile: two 32-key blocks. hi = false (the tail tile when
// its second block holds no real key): block 1 is not multiplied and its
// scores are -inf, as the mask would make them.
template <int D>
__device__ __forceinline__ void qk_tile(const char *kt, int kx, const bf16x8 *qop, f32x16 *sacc, bool hi = true) {
  constexpr int DK = D / 16;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk == 1 && !hi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[1][r] = -INFINITY;
      break;
    }
    sacc[blk] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kt + blk * 32 * D * 2 + (kx ^ (32 * dk)));
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
  uint32_t wbase;
  const bf16_t *kbase, *vbase;
  const int *koff, *voff;
  int kx, vx;
  const bf16x8 *qop;
  int ks_bytes, vs_bytes, kv_valid, t_end, wave, hf;
  float c2;
};

// One key tile of the main loop: S(t+1) = K(t+1) Q^T and O^T += V(t)^T
// P(t)^T on the matrix cores, with the VALU work spread over both MFMA
// groups (3 VALU ops per S MFMA, 4 per P.V MFMA): P(t) = exp2(S(t) - m) for
// key block 0 runs beside S(t+1), block 1 beside the P.V of block 0, and
// the row max of S(t+1) beside the rest. Then the (rare) lazy rescale.
// par is the LDS buffer parity of tile t within the current key range.
// STEADY: tile t+1 exists and is full, parity static, scheduled with
// sched_group_barrier. Otherwise has_next / mask_next are run-time flags
// (the last tiles of a run) and the next scores are copied into scur.
// FIXED: the row maximum is the fixed-m bound (no running max, no rescale).
template <int D, bool STEADY, bool FIXED>
__device__ __forceinline__ void step(const StepCtx<D> &cx, int t, int par, f32x16 *scur, f32x16 *snext,
                                     f32x16 *acc_o, float &m_run, float &l_run, bool has_next = true,
                                     bool mask_next = false) {
  const bool HAS_NEXT = STEADY || has_next;
  using G = Geo<D>;
  const int kx = cx.kx, vx = cx.vx;
  constexpr int DK = D / 16, DB = D / 32;
  if (t + 2 < cx.t_end)
    issue_rows_par<D, G::K0>(par, cx.wbase, cx.kbase, cx.ks_bytes, t + 2, cx.kv_valid, cx.koff);
  if (HAS_NEXT)
    issue_rows_par<D, G::V0>(par ^ 1, cx.wbase, cx.vbase, cx.vs_bytes, t + 1, cx.kv_valid, cx.voff);
  debug_sync();
  const char *vt = cx.smem + G::V0 + par * G::TILE_BYTES;

  const float neg_m = -m_run;
  bf16x8 pop[2][2];
  float ps0 = 0.f, ps1 = 0.f;
  auto softmax_block = [&](int blk) {
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
  };
  // tail tiles only: whether the second 32-key block of tile t (cur_hi) or
  // of tile t+1 (next_hi) holds a real key; an empty block contributes
  // p = 0 exactly, so its exp2, MFMAs and sums are skipped
  const bool cur_hi = STEADY || t * BN + 32 < cx.kv_valid;
  const bool next_hi = STEADY || !mask_next || (t + 1) * BN + 32 < cx.kv_valid;
  softmax_block(0);
  if (HAS_NEXT) {
    qk_tile<D>(cx.smem + G::K0 + (par ^ 1) * G::TILE_BYTES, kx, cx.qop, snext, next_hi);
    if (!STEADY && mask_next) mask_tail(snext, (t + 1) * BN, cx.kv_valid, cx.hf);
  }
  debug_sync();
  if (cur_hi) softmax_block(1);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk == 1 && !cur_hi) break;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const char *src = vt + (blk * 32 + a * 16) * D * 2 + (vx ^ (64 * db));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(src));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(src + 4 * D * 2));
        const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pop[blk][a], acc_o[db], 0, 0, 0);
      }
    }
  }
  debug_sync();
  float mts = 0.f;
  if (!FIXED && HAS_NEXT) mts = pair_max(snext) * cx.c2;
  if (STEADY) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * DK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  }
  l_run += ps0 + ps1;

  if (HAS_NEXT) {
    const bool upd = !FIXED && mts > m_run + kLazyRescale;
    if (!FIXED && __any(upd)) {
      const float m_new = upd ? mts : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
    if (!STEADY) {
      scur[0] = snext[0];
      scur[1] = snext[1];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
}

// Per-workgroup state that does not depend on which q-tile is processed.
template <int D>
struct Lane {
  int tid, lane, wave, l32, hf;
  int ks_bytes, vs_bytes;
  int koff[Geo<D>::LOADS_PER_WAVE], voff[Geo<D>::LOADS_PER_WAVE];
  int kx, vx;   // operand read offsets of d-chunk 0 (see the kernel prologue)
};

// Q operand (B of S^T) of this lane: query qrow of the q-tile, channel
// d = dk*16 + hf*8 + e; rows past s_q load as zeros.
template <int D, class P>
__device__ __forceinline__ void load_q(const P &p, const Lane<D> &ln, int b, int h, int qt, bf16x8 *qop) {
  constexpr int DK = D / 16;
  const bf16_t *qbase = p.q + b * p.qs_b + h * p.qs_h;
  const int qrow = qt * BM + ln.wave * 32 + ln.l32;
  u32x4 raw[DK];
  const bool in_q = qrow < p.s_q;
  const bf16_t *qr = qbase + (int64_t)(in_q ? qrow : 0) * p.qs_s;
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) raw[dk] = in_q ? ldg16(qr + dk * 16 + ln.hf * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) qop[dk] = __builtin_bit_cast(bf16x8, raw[dk]);
}

// Whether query row qrow is a real token: q_valid counts the real rows of
// the whole sequence, or of each q_seg_len-row segment when q_seg_len > 0.
template <class P>
__device__ __forceinline__ bool query_is_real(const P &p, int qrow) {
  return p.q_seg_len > 0 ? (qrow < p.s_q && qrow % p.q_seg_len < p.q_valid) : qrow < p.q_valid;
}

// Whether any of the 32 rows r0 .. r0 + 31 of a wave is real, from
// wave-uniform values only (so the branch on it stays uniform). With
// segments: either r0 itself is real, or the first row of the next segment
// lies in the range (it is real whenever q_valid > 0).
template <class P>
__device__ __forceinline__ bool wave_has_real_row(const P &p, int r0) {
  if (p.q_seg_len == 0) return r0 < p.q_valid;
  const int end = r0 + 32 < p.s_q ? r0 + 32 : p.s_q;
  if (r0 >= end || p.q_valid == 0) return false;
  const int off = r0 % p.q_seg_len;
  return off < p.q_valid || r0 - off + p.q_seg_len < end;
}

// Attention of one q-tile (BM rows of head (b, h)) over the key tiles
// [kb, ke), whose rows at or past kv_end are pads (they are fetched as zeros
// and masked). FIRST: the first key range of the q-tile: Q is loaded into
// qop (while the first K/V tiles are in flight) and the running state starts
// from this range; otherwise qop is already loaded and the range continues
// the running state (a raised maximum rescales O and l). On return acc_o
// holds this lane's unnormalised O^T (query qrow), m_run the running max
// (log2 units, scaled) and l_run this lane's half of the row sum.
// FIXED: the running maximum is the q-tile's fixed-m bound, loaded with Q
// (the range never raises it).
template <int D, bool FIRST, bool FIXED, class P>
__device__ __forceinline__ void run_keys(const P &p, char *smem, const Lane<D> &ln, int b, int h, int qt, int kb,
                                         int ke, int kv_end, bf16x8 *qop, f32x16 *acc_o, float &m_run,
                                         float &l_run) {
  using G = Geo<D>;
  constexpr int DB = D / 32;
  const bf16_t *kbase = p.k + b * p.ks_b + h * p.ks_h;
  const bf16_t *vbase = p.v + b * p.vs_b + h * p.vs_h;

  const uint32_t wbase = (uint32_t)(uintptr_t)(lds_void_t *)smem + ln.wave * G::LOADS_PER_WAVE * 1024;
  issue_rows<D, G::K0>(wbase, kbase, ln.ks_bytes, kb, kv_end, ln.koff);
  issue_rows<D, G::V0>(wbase, vbase, ln.vs_bytes, kb, kv_end, ln.voff);
  if (kb + 1 < ke) issue_rows<D, G::K0 + G::TILE_BYTES>(wbase, kbase, ln.ks_bytes, kb + 1, kv_end, ln.koff);
  debug_sync();

  // a wave whose 32 query rows are all pads (tail pads of the sequence or
  // of their segments, or rows past s_q) does no arithmetic: it still
  // issues its share of every K/V tile and meets the others at each
  // barrier, and its rows are written as pads
  if (!wave_has_real_row(p, qt * BM + ln.wave * 32)) {
    if (FIRST) {
      l_run = 0.f;
      m_run = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    __syncthreads();
    for (int t = kb; t < ke; ++t) {
      const int par = (t - kb) & 1;
      if (t + 2 < ke) issue_rows_par<D, G::K0>(par, wbase, kbase, ln.ks_bytes, t + 2, kv_end, ln.koff);
      if (t + 1 < ke) issue_rows_par<D, G::V0>(par ^ 1, wbase, vbase, ln.vs_bytes, t + 1, kv_end, ln.voff);
      debug_sync();
      debug_sync();
      debug_sync();
      if (t + 1 < ke) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
    }
    return;
  }

  float m_fix = 0.f;
  if (FIRST) {
    load_q<D>(p, ln, b, h, qt, qop);
    if (FIXED) {
      const int qrow = qt * BM + ln.wave * 32 + ln.l32;
      m_fix = qrow < p.s_q ? p.fm_m[((int64_t)b * p.H + h) * p.s_q + qrow] : 0.f;
    }
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};
  }
  const float c2 = p.scale_log2;
  f32x16 sa[2], sb[2];
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K(kb), V(kb), K(kb+1) landed
  __syncthreads();
  qk_tile<D>(smem + G::K0, ln.kx, qop, sa);
  __syncthreads();                      // K(kb)'s buffer is refilled by the first step
  if ((kb + 1) * BN > kv_end) mask_tail(sa, kb * BN, kv_end, ln.hf);
  if (FIXED) {
    if (FIRST) m_run = m_fix;
  } else if (FIRST) {
    m_run = pair_max(sa) * c2;          // first tile: nothing accumulated yet
  } else {
    const float mt = pair_max(sa) * c2;
    const bool upd = mt > m_run + kLazyRescale;
    if (__any(upd)) {
      const float m_new = upd ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
  }

  if (FIRST) clock_mark(0);
  StepCtx<D> cx{smem, wbase, kbase, vbase, ln.koff, ln.voff, ln.kx, ln.vx, qop,
                ln.ks_bytes, ln.vs_bytes, kv_end, ke, ln.wave, ln.hf, c2};
  // steady state: tiles t, t+1, t+2 all full; two tiles per iteration so the
  // score registers alternate roles and the LDS buffer parity is static
  int t = kb;
  for (; t + 3 < ke; t += 2) {
    step<D, true, FIXED>(cx, t, 0, sa, sb, acc_o, m_run, l_run);
    step<D, true, FIXED>(cx, t + 1, 1, sb, sa, acc_o, m_run, l_run);
  }
  // the last (at most three) tiles: run-time flags; tile t+1 may be the
  // masked tail
  for (; t < ke; ++t) {
    const bool has_next = t + 1 < ke;
    step<D, false, FIXED>(cx, t, (t - kb) & 1, sa, sb, acc_o, m_run, l_run, has_next,
                          has_next && (t + 2) * BN > kv_end);
  }
}

// One q-tile over the key tiles [kb, ke) of a key range whose real rows end
// at kv_valid.
template <int D, class P>
__device__ __forceinline__ void run_qtile(const P &p, char *smem, const Lane<D> &ln, int b, int h, int qt,
                                          int kb, int ke, f32x16 *acc_o, float &m_run, float &l_run) {
  bf16x8 qop[D / 16];
  run_keys<D, true, false>(p, smem, ln, b, h, qt, kb, ke, p.kv_valid, qop, acc_o, m_run, l_run);
}

// Whether q-tile qt of head (b, h) runs with the fixed-m bound (set up and
// found tight enough by launch_fixed_m); uniform over the workgroup.
template <class P>
__device__ __forceinline__ bool use_fixed_m(const P &p, int b, int h, int qt) {
  return p.fm_m != nullptr && p.fm_ok[((int64_t)b * p.H + h) * p.n_qtiles + qt] != 0;
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Final epilogue: O = acc / l; LSE = (m + log2 l) ln 2; pad rows by select.
template <int D, class P>
__device__ __forceinline__ void store_final(const P &p, int b, int h, int qrow, int hf, const f32x16 *acc_o,
                                            float lse2, float inv_l, bool row_ok) {
  constexpr int DB = D / 32;
  if (qrow >= p.s_q) return;
  const int64_t obase = b * p.os_b + h * p.os_h + (int64_t)qrow * p.os_s;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + 8 * i + 4 * hf;
      float o4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o4[j] = row_ok ? acc_o[db][4 * i + j] * inv_l : 0.0f;
      if (p.o_f32) {
        float *op = reinterpret_cast<float *>(p.o) + obase + d0;
        *reinterpret_cast<float4 *>(op) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      } else {
        bf16_t *op = reinterpret_cast<bf16_t *>(p.o) + obase + d0;
        *reinterpret_cast<u32x2 *>(op) = u32x2{pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
      }
    }
  }
  if (p.lse != nullptr && hf == 0) p.lse[((int64_t)b * p.H + h) * p.s_q + qrow] = row_ok ? lse2 * kLn2 : -INFINITY;
}

// Final epilogue of a whole q-tile with bf16 O, staged through LDS: each
// wave writes its 32 x D block of O into its own slice of the tile buffers
// (idle once every wave has finished the last tile), then reads it back so
// that 16 lanes hold one row's D * 2 contiguous bytes and every store
// instruction writes whole rows, instead of 16-byte pieces of 32 rows. The
// 16-byte chunks of a row sit XOR-swizzled by the row in LDS; the 8 KB
// each wave writes and reads back cost 64 bank-conflict cycles per wave
// (SQ_LDS_BANK_CONFLICT), small next to the stores this saves. Pad rows
// are written as 0 and their LSE as -inf; rows past s_q are not written.
// All threads of the workgroup must call it (it has a barrier).
template <int D, class P>
__device__ __forceinline__ void store_final_staged(const P &p, char *smem, const Lane<D> &ln, int b, int h, int qt,
                                                   const f32x16 *acc_o, float lse2, float inv_l, bool row_ok) {
  constexpr int DB = D / 32, CPR = D / 8, ROWB = D * 2;
  char *slice = smem + ln.wave * (32 * ROWB);
  __syncthreads();   // every wave is done reading the last K / V tiles
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // this lane's channels db*32 + 8i + 4hf .. +3 of row l32: chunk db*4 + i
      const int j = db * 4 + i;
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = row_ok ? acc_o[db][4 * i + e] * inv_l : 0.0f;
      *reinterpret_cast<u32x2 *>(slice + ln.l32 * ROWB + ((j ^ (ln.l32 % CPR)) * 16) + ln.hf * 8) =
          u32x2{pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3])};
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const int row0 = qt * BM + ln.wave * 32;
  bf16_t *obase = reinterpret_cast<bf16_t *>(p.o) + b * p.os_b + h * p.os_h;
#pragma unroll
  for (int k = 0; k < 32 * CPR / 64; ++k) {
    const int c = k * 64 + ln.lane;
    const int r = c / CPR, j = c % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(slice + r * ROWB + ((j ^ (r % CPR)) * 16));
    if (row0 + r < p.s_q) *reinterpret_cast<u32x4 *>(obase + (int64_t)(row0 + r) * p.os_s + j * 8) = v;
  }
  const int qrow = row0 + ln.l32;
  if (p.lse != nullptr && ln.hf == 0 && qrow < p.s_q)
    p.lse[((int64_t)b * p.H + h) * p.s_q + qrow] = row_ok ? lse2 * kLn2 : -INFINITY;
}

// Partials of split q-tiles move between workgroups that may sit on
// different XCDs (separate L2s), so they are written and read with the
// device-scope cache policy (sc1): such a store is complete at the device's
// coherence point once vmcnt reaches zero, and such a load is served from
// it, so no whole-L2 writeback or invalidate is needed. Slot s holds 512
// threads x (d/8) float4 of O / l, stored chunk-major so one wave
// instruction covers 1 KB contiguously, and 256 floats of log2 LSE.
constexpr int kSC1 = 16;   // buffer cache-policy bit: device scope

template <int D, class P>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_o_view(const P &p, int slot) {
  constexpr int BYTES = NT * D * 2;   // NT threads x (D/2) floats
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char *>(p.sk_part_o) + (int64_t)slot * BYTES, 0, BYTES,
                                           0x00020000);
}

template <class P>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_l_view(const P &p, int slot) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char *>(p.sk_part_l) + (int64_t)slot * BM * 4, 0, BM * 4,
                                           0x00020000);
}

// Split-schedule geometry ("data-parallel + Stream-K tail"). With M > 0,
// main workgroup T < M (= the number of q-tiles) runs keys [0, kc) of
// q-tile T, all of them in step so each K/V tile is read while it is in L2;
// the H helper workgroups split the remaining tails [kc, nk) of all q-tiles,
// flattened q-tile major into U = nq (nk - kc) units, into equal contiguous
// ranges (helper h owns [h U / H, (h+1) U / H)). With M = 0 and kc = 0 this
// is plain Stream-K over every unit. Partial-result slots: main T uses slot
// T; helper slots as in helper_slot.
struct SkGeo {
  int64_t U;
  int M, H, nk, kc;
  __device__ int nt() const { return nk - kc; }
  __device__ int64_t start(int h) const { return (int64_t)h * U / H; }
  // the helper whose range holds tail unit u
  __device__ int owner(int64_t u) const { return (int)(((u + 1) * H - 1) / U); }
  __device__ int helper_slot(int h, int T) const {
    // with main workgroups, a helper's middle q-tiles are pieces too: slot
    // M + h + T is unique (helper h's q-tiles start at or after helper
    // h-1's last) and below M + H + nq <= 2 grid; without them (plain
    // Stream-K) a middle q-tile is whole and two slots per helper suffice
    return M > 0 ? M + h + T : 2 * h + ((int)(start(h) / nt()) == T ? 0 : 1);
  }
  // q-tile T's pieces in key order: piece 0 is the main workgroup's (when
  // M > 0), then the helpers h_lo(T)..h_hi(T)
  __device__ int h_lo(int T) const { return owner((int64_t)T * nt()); }
  __device__ int h_hi(int T) const { return owner((int64_t)(T + 1) * nt() - 1); }
  __device__ int n_pieces(int T) const { return (M > 0 ? 1 : 0) + h_hi(T) - h_lo(T) + 1; }
  __device__ int slot_of_piece(int T, int x) const {
    if (M > 0) {
      if (x == 0) return T;
      --x;
    }
    return helper_slot(h_lo(T) + x, T);
  }
};

// Store this workgroup's piece of q-tile T (o = acc / l, normalised, and
// its log2 LSE) into `slot`, device-scope.
template <int D, class P>
__device__ __forceinline__ void store_piece(const P &p, const Lane<D> &ln, int slot, const f32x16 *o, float lse2) {
  constexpr int DB = D / 32;
  const __amdgpu_buffer_rsrc_t v = part_o_view<D>(p, slot);
#pragma unroll
  for (int j = 0; j < DB * 4; ++j) {
    const int db = j >> 2, r = 4 * (j & 3);
    const u32x4 c = {__float_as_uint(o[db][r]), __float_as_uint(o[db][r + 1]), __float_as_uint(o[db][r + 2]),
                     __float_as_uint(o[db][r + 3])};
    __builtin_amdgcn_raw_buffer_store_b128(c, v, ln.tid * 16, j * NT * 16, kSC1);
  }
  if (ln.hf == 0)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2), part_l_view(p, slot), (ln.wave * 32 + ln.l32) * 4, 0,
                                          kSC1);
}

// The last piece of q-tile T to finish combines its n pieces (this
// workgroup's own piece, index `own`, is still in registers as the
// normalised o = acc / l with log2 LSE lse2; o is overwritten) and writes
// the final O and LSE: O = sum_s w_s o_s / sum_s w_s with
// w_s = 2^(lse_s - M), M = max_s lse_s, summed in key order whichever piece
// finished last, so the result is the same bits on every call. Up to
// kFastPieces pieces the loads are batched (every LSE at once; the other
// pieces' share of one 32-channel block at once), so the merge costs one
// memory round trip per 32-channel block plus one; beyond that a plain loop.
constexpr int kFastPieces = 4;

template <int D, class P>
__device__ __forceinline__ void merge_pieces(const P &p, const Lane<D> &ln, const SkGeo &sk, int T, int own, int b,
                                             int h, int qrow, bool row_ok, f32x16 *o, float lse2) {
  constexpr int DB = D / 32;
  constexpr int KO = kFastPieces - 1;   // other pieces on the fast path
  const int row = ln.wave * 32 + ln.l32;
  const int n = sk.n_pieces(T);
  float M = lse2, wsum = 0.f;
  if (n <= kFastPieces) {
    // the other pieces in key order: oth[k] is piece x_k (k < n - 1)
    int slot[KO];
    float lx[KO], wx[KO];
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int x = k < own ? k : k + 1;
      slot[k] = k < n - 1 ? sk.slot_of_piece(T, x) : 0;
      lx[k] = k < n - 1 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(part_l_view(p, slot[k]), row * 4, 0,
                                                                              kSC1))
                        : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < KO; ++k) M = fmaxf(M, lx[k]);
    const float w_own = __builtin_amdgcn_exp2f(lse2 - M);
    // the sum of weights in key order: pieces before own, own, after own
    for (int x = 0; x < n; ++x) {
      const int k = x < own ? x : x - 1;
      float w = 0.f;
#pragma unroll
      for (int kk = 0; kk < KO; ++kk) w = kk == k ? __builtin_amdgcn_exp2f(lx[kk] - M) : w;
      wsum += x == own ? w_own : w;
    }
#pragma unroll
    for (int k = 0; k < KO; ++k) wx[k] = k < n - 1 ? __builtin_amdgcn_exp2f(lx[k] - M) : 0.f;
    auto load_block = [&](int db, u32x4 (&c)[KO][4]) {
#pragma unroll
      for (int k = 0; k < KO; ++k) {
        if (k < n - 1) {
          const __amdgpu_buffer_rsrc_t v = part_o_view<D>(p, slot[k]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            c[k][i] = __builtin_amdgcn_raw_buffer_load_b128(v, ln.tid * 16, (db * 4 + i) * NT * 16, kSC1);
        }
      }
    };
    u32x4 cur[KO][4];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      load_block(db, cur);
      f32x16 a = f32x16{};
      // key order: the other pieces before own, own, the ones after
      for (int x = 0; x < n; ++x) {
        if (x == own) {
#pragma unroll
          for (int r = 0; r < 16; ++r) a[r] = fmaf(w_own, o[db][r], a[r]);
        } else {
          const int k = x < own ? x : x - 1;
#pragma unroll
          for (int kk = 0; kk < KO; ++kk) {
            if (kk == k) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * i + e] = fmaf(wx[kk], __uint_as_float(cur[kk][i][e]), a[4 * i + e]);
            }
          }
        }
      }
      o[db] = a;
    }
  } else {
    auto lse_of = [&](int x) {
      return x == own ? lse2
                      : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(part_l_view(p, sk.slot_of_piece(T, x)),
                                                                             row * 4, 0, kSC1));
    };
    M = -INFINITY;
    for (int x = 0; x < n; ++x) M = fmaxf(M, lse_of(x));
    for (int x = 0; x < n; ++x) wsum += __builtin_amdgcn_exp2f(lse_of(x) - M);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x16 a = f32x16{};
      for (int x = 0; x < n; ++x) {
        const float w = __builtin_amdgcn_exp2f(lse_of(x) - M);
        if (x == own) {
#pragma unroll
          for (int r = 0; r < 16; ++r) a[r] = fmaf(w, o[db][r], a[r]);
        } else {
          const __amdgpu_buffer_rsrc_t v = part_o_view<D>(p, sk.slot_of_piece(T, x));
          u32x4 c[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            c[i] = __builtin_amdgcn_raw_buffer_load_b128(v, ln.tid * 16, (db * 4 + i) * NT * 16, kSC1);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * i + e] = fmaf(w, __uint_as_float(c[i][e]), a[4 * i + e]);
        }
      }
      o[db] = a;
    }
  }
  store_final<D>(p, b, h, qrow, ln.hf, o, M + __log2f(wsum), row_ok ? 1.0f / wsum : 0.f, row_ok);
}

// Per-lane constants: wave / lane ids, the DMA source offsets and the
// operand read offsets.
template <int D, class P>
__device__ __forceinline__ void make_lane(const P &p, int tid, Lane<D> &ln) {
  using G = Geo<D>;
  constexpr int CPR = G::CPR;
  ln.tid = tid;
  ln.lane = ln.tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.l32 = ln.lane & 31;
  ln.hf = ln.lane >> 5;
  ln.ks_bytes = (int)(p.ks_s * 2);
  ln.vs_bytes = (int)(p.vs_s * 2);
  // Per-lane source offsets for the wave's share of a tile: load i of wave w
  // fills LDS slots s = (w*LPW + i)*64 + lane (16 bytes each), i.e. row
  // s / CPR, position s % CPR, which holds chunk (position ^ f(row)).
#pragma unroll
  for (int i = 0; i < G::LOADS_PER_WAVE; ++i) {
    const int s = (ln.wave * G::LOADS_PER_WAVE + i) * 64 + ln.lane;
    const int r = s / CPR, pos = s % CPR;
    ln.koff[i] = r * ln.ks_bytes + ((pos ^ G::fk(r)) * 16);
    ln.voff[i] = r * ln.vs_bytes + ((pos ^ G::fv(r)) * 16);
  }
  // K operand: MFMA row m = l32 of block blk holds key blk*32 + kperm
  const int kperm = (ln.l32 & 16) + ((ln.l32 & 4) << 1) + ((ln.l32 & 8) >> 1) + (ln.l32 & 3);
  // chunk 2*dk + hf of row kperm sits at position (2*dk + hf) ^ fk(kperm);
  // the row offset and (hf ^ fk) * 16 occupy bits disjoint from 32 * dk, so
  // the offset for d-chunk dk is kx ^ (32 * dk)
  ln.kx = kperm * (D * 2) + ((ln.hf ^ G::fk(kperm)) * 16);
  // V operand via transpose reads: lane 16g + 4e + q points at
  // V[base + 8*(g>>1) + e][db*32 + 16*(g&1) + 4q]
  {
    const int tg = ln.lane >> 4, te = (ln.lane >> 2) & 3, tq = ln.lane & 3;
    const int vrow = 8 * (tg >> 1) + te;
    // chunk 4*db + c0 (c0 < 4) sits at position chunk ^ fv(vrow), fv a
    // multiple of 4, so the offset for channel block db is vx ^ (64 * db)
    const int chunk0 = 2 * (tg & 1) + (tq >> 1);
    ln.vx = vrow * (D * 2) + ((chunk0 ^ G::fv(vrow)) * 16) + 8 * (tq & 1);
  }
}

// Dynamic placement of whole q-tiles: the q-tiles, in (b, h, tile) order,
// form eight contiguous queues, queue x holding the tiles the static
// placement puts on XCD x (so a queue's tiles share K / V in that XCD's L2);
// workgroup i runs on XCD i % 8 (round-robin dispatch). The first
// p.dyn_static workgroups (one wave: one per CU) take the head of their own
// XCD's queue by index, with no atomics, so a launch does not start with
// hundreds of workgroups contending for eight counters. Every later
// workgroup takes the next tile of its own queue, else of the others in
// turn, through the device-scope counters sk_count[0..7] (counting past the
// static part); -1 when every queue is empty. The grid has spare
// workgroups: the XCDs run at their own clocks under the power limit, and
// those that get through their queue first take over tiles the slower ones
// have not started. The last of the later workgroups to take (counted in
// sk_count[8]) sets the nine counters back to zero for the next call.
// Uniform over the workgroup (sh: a shared int for the broadcast).
constexpr int kDynQueues = 8;

template <class P>
__device__ __forceinline__ int take_tile(const P &p, int &sh) {
  const int total = p.n_qtiles * p.H * p.B;
  const int q8 = total / kDynQueues, r8 = total % kDynQueues;
  const int S = p.dyn_static;
  const int bid = (int)blockIdx.x;
  if (bid < S) {   // first wave: the head of its own queue, by index
    const int x = bid % kDynQueues, idx = bid / kDynQueues;
    const int start = x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8;
    const int len = q8 + (x < r8 ? 1 : 0);
    return idx < len ? start + idx : -1;
  }
  if (threadIdx.x == 0) {
    int t = -1;
    for (int k = 0; k < kDynQueues && t < 0; ++k) {
      const int x = (bid + k) % kDynQueues;
      const int start = x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8;
      const int len = q8 + (x < r8 ? 1 : 0);
      const int n_static = x < S ? (S - x + kDynQueues - 1) / kDynQueues : 0;   // taken by index
      const int base = n_static < len ? n_static : len;
      const int i = __hip_atomic_fetch_add(p.sk_count + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (i >= 0 && base + i < len) t = start + base + i;   // (i < 0 only if a caller broke the zero-counter contract)
    }
    const int taken =
        __hip_atomic_fetch_add(p.sk_count + kDynQueues, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (taken == (int)gridDim.x - S - 1) {   // every other later workgroup has taken its tile (or found none)
      for (int x = 0; x <= kDynQueues; ++x)
        __hip_atomic_store(p.sk_count + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sh = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(sh);
}

template <int D, bool STREAMK, bool DYN = false>
__global__ __launch_bounds__(NT, 512 / NT) void attn_fwd_kernel(AttnParams p) {
  using G = Geo<D>;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[4 * G::TILE_BYTES];
  __shared__ int last_flag;

  if (!STREAMK) clock_edge(0);
  Lane<D> ln;
  make_lane<D>(p, threadIdx.x, ln);

  const int kv_valid = p.kv_valid;
  const int nk = (kv_valid + BN - 1) / BN;
  f32x16 acc_o[DB];
  float m_run = -INFINITY, l_run = 0.f;

  if (!STREAMK) {
    // one workgroup per q-tile, all key tiles; the q-tile is placed by the
    // block index, or taken from the dynamic queues
    int logical;
    if (DYN) {
      logical = take_tile(p, last_flag);
      if (logical < 0) return;   // uniform: every queue was empty
    } else {
      logical = xcd_remap(blockIdx.x, gridDim.x);
    }
    const int qt = logical % p.n_qtiles;
    const int bh = logical / p.n_qtiles;
    const int h = bh % p.H, b = bh / p.H;
    const int qrow = qt * BM + ln.wave * 32 + ln.l32;
    if (nk > 0) {
      bf16x8 qop[D / 16];
      if (use_fixed_m(p, b, h, qt))
        run_keys<D, true, true>(p, smem, ln, b, h, qt, 0, nk, p.kv_valid, qop, acc_o, m_run, l_run);
      else
        run_keys<D, true, false>(p, smem, ln, b, h, qt, 0, nk, p.kv_valid, qop, acc_o, m_run, l_run);
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};
    }
    clock_mark(1);
    clock_note_tiles(nk);
    const float l_tot = pair_sum(l_run);
    const bool row_ok = query_is_real(p, qrow) && (nk > 0);
    if (p.o_f32)
      store_final<D>(p, b, h, qrow, ln.hf, acc_o, m_run + __log2f(l_tot), row_ok ? 1.0f / l_tot : 0.f, row_ok);
    else
      store_final_staged<D>(p, smem, ln, b, h, qt, acc_o, m_run + __log2f(l_tot), row_ok ? 1.0f / l_tot : 0.f,
                            row_ok);
    clock_edge(1);
    return;
  }

  // ---- split schedule (geometry in SkGeo): a main workgroup runs one
  // piece, a helper the pieces of its range in order. A piece covering a
  // whole q-tile writes the final result; any other piece writes its
  // partial (device scope) and, once every thread's stores have completed,
  // bumps the q-tile's arrival counter; the piece that arrives last merges
  // all pieces. Logical workgroups are contiguous per XCD, so the main
  // workgroups of one head (one K/V) share an XCD's L2.
  const int nq_all = p.n_qtiles * p.H * p.B;
  const SkGeo sk{(int64_t)nq_all * (nk - p.sk_kc), p.sk_main, p.sk_grid - p.sk_main, nk, p.sk_kc};
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  int64_t u, u_end;
  int hh = -1;   // helper index, or -1 for a main workgroup
  if (g < sk.M) {
    u = (int64_t)g * nk;   // main: q-tile g, keys [0, kc)
    u_end = u + sk.kc;
  } else {
    hh = g - sk.M;
    u = sk.start(hh);
    u_end = sk.start(hh + 1);
  }
  while (u < u_end) {
    int T, kb, ke;
    if (hh < 0) {
      T = g;
      kb = 0;
      ke = sk.kc;
    } else {
      T = (int)(u / sk.nt());
      kb = sk.kc + (int)(u - (int64_t)T * sk.nt());
      ke = (int)((int64_t)kb + (u_end - u) < nk ? (int64_t)kb + (u_end - u) : nk);
    }
    const int qt = T % p.n_qtiles, bh = T / p.n_qtiles;
    const int h = bh % p.H, b = bh / p.H;
    const int qrow = qt * BM + ln.wave * 32 + ln.l32;
    run_qtile<D>(p, smem, ln, b, h, qt, kb, ke, acc_o, m_run, l_run);
    clock_mark(1);
    clock_note_tiles(ke - kb);
    const float l_tot = pair_sum(l_run);
    const float lse2 = m_run + __log2f(l_tot);
    const bool row_ok = query_is_real(p, qrow);
    if (kb == 0 && ke == nk) {
      store_final<D>(p, b, h, qrow, ln.hf, acc_o, lse2, row_ok ? 1.0f / l_tot : 0.f, row_ok);
    } else {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= inv;
      const int own = hh < 0 ? 0 : (sk.M > 0 ? 1 : 0) + hh - sk.h_lo(T);
      const int np = sk.n_pieces(T);
      // if every other piece has already arrived (each publishes before it
      // counts itself), this one is last: merge without publishing
      if (ln.tid == 0) {
        const int seen = __hip_atomic_load(p.sk_count + T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = seen == np - 1 ? 1 : 0;
        if (last_flag) __hip_atomic_store(p.sk_count + T, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (!last_flag) {
        store_piece<D>(p, ln, sk.slot_of_piece(T, own), acc_o, lse2);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's piece is at the coherence point
        __syncthreads();                      // ... and every other thread's (and last_flag was read)
        if (ln.tid == 0) {
          const int old = __hip_atomic_fetch_add(p.sk_count + T, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last_flag = (old == np - 1) ? 1 : 0;
          if (last_flag) __hip_atomic_store(p.sk_count + T, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
      }
      if (last_flag) merge_pieces<D>(p, ln, sk, T, own, b, h, qrow, row_ok, acc_o, lse2);
    }
    u += ke - kb;
    __syncthreads();   // every wave is done with this piece's LDS tiles and last_flag
  }
}

// Keys in n_kv_seg segments of kv_seg_len rows (a multiple of the key tile),
// each holding kv_valid real rows followed by its own tail pad (the ring
// layout of maxdiffusion PR #491, each ring segment padded at its own tail):
// one workgroup per q-tile runs the key tiles of every segment's real rows in
// turn, continuing one online softmax, so the result is the softmax over the
// union of the real keys.
template <int D>
__global__ __launch_bounds__(NT, 512 / NT) void attn_fwd_seg_kernel(AttnParams p) {
  using G = Geo<D>;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[4 * G::TILE_BYTES];

  Lane<D> ln;
  make_lane<D>(p, threadIdx.x, ln);
  const int tps = (p.kv_valid + BN - 1) / BN;   // key tiles with real rows, per segment
  const int seg_tiles = p.kv_seg_len / BN;
  f32x16 acc_o[DB];
  float m_run = -INFINITY, l_run = 0.f;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;
  const int h = bh % p.H, b = bh / p.H;
  const int qrow = qt * BM + ln.wave * 32 + ln.l32;
  if (tps > 0) {
    bf16x8 qop[D / 16];
    if (use_fixed_m(p, b, h, qt)) {
      run_keys<D, true, true>(p, smem, ln, b, h, qt, 0, tps, p.kv_valid, qop, acc_o, m_run, l_run);
      for (int sg = 1; sg < p.n_kv_seg; ++sg) {
        __syncthreads();   // every wave is done with the previous range's LDS tiles
        const int kb = sg * seg_tiles;
        run_keys<D, false, true>(p, smem, ln, b, h, qt, kb, kb + tps, sg * p.kv_seg_len + p.kv_valid, qop, acc_o,
                                 m_run, l_run);
      }
    } else {
      run_keys<D, true, false>(p, smem, ln, b, h, qt, 0, tps, p.kv_valid, qop, acc_o, m_run, l_run);
      for (int sg = 1; sg < p.n_kv_seg; ++sg) {
        __syncthreads();   // every wave is done with the previous range's LDS tiles
        const int kb = sg * seg_tiles;
        run_keys<D, false, false>(p, smem, ln, b, h, qt, kb, kb + tps, sg * p.kv_seg_len + p.kv_valid, qop, acc_o,
                                  m_run, l_run);
      }
    }
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};
  }
  const float l_tot = pair_sum(l_run);
  const bool row_ok = query_is_real(p, qrow) && (tps > 0);
  if (p.o_f32)
    store_final<D>(p, b, h, qrow, ln.hf, acc_o, m_run + __log2f(l_tot), row_ok ? 1.0f / l_tot : 0.f, row_ok);
  else
    store_final_staged<D>(p, smem, ln, b, h, qt, acc_o, m_run + __log2f(l_tot), row_ok ? 1.0f / l_tot : 0.f,
                          row_ok);
}

// Pre-pass of Q and K (blockIdx.y picks the tensor): optional per-head RMS
// normalisation with weights, then optional split-halves rotation, in fp32
// from the bf16 input, rounded once to bf16. A thread owns one 8-channel run
// of the first half of a row and its partner run d/2 later: it loads that
// row's 16 table values once and applies them to the row of up to
// kRopeHeads (b, h) pairs (blockIdx.z picks the group), so the tables are
// read once per row and head group rather than once per head. The RMS of a
// head vector is summed over the RUNS = d/16 consecutive lanes of its row.
// The first workgroup also clears the Stream-K arrival counters of the
// attention launch that follows (saving that launch a clearing kernel).
constexpr int kRopeHeads = 4;

template <int RUNS>
__global__ __launch_bounds__(256) void rope_rotate_kernel(RopeRotateParams p) {
  constexpr int ROWS = 256 / RUNS, HALF = RUNS * 8;
  const RopeSeg &g = p.seg[blockIdx.y];
  if (p.zero != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < p.n_zero; i += 256) p.zero[i] = 0;
  const int c = threadIdx.x % RUNS;
  const int nbh = p.B * p.H;
  const int bh0 = blockIdx.z * kRopeHeads;
  const int nh = nbh - bh0 < kRopeHeads ? nbh - bh0 : kRopeHeads;
  const bool rot = g.cos_t != nullptr, nrm = g.norm_w != nullptr;
  float w1[8], w2[8];
  if (nrm) {
    const float4 a0 = *reinterpret_cast<const float4 *>(g.norm_w + c * 8);
    const float4 a1 = *reinterpret_cast<const float4 *>(g.norm_w + c * 8 + 4);
    const float4 b0 = *reinterpret_cast<const float4 *>(g.norm_w + HALF + c * 8);
    const float4 b1 = *reinterpret_cast<const float4 *>(g.norm_w + HALF + c * 8 + 4);
    w1[0] = a0.x; w1[1] = a0.y; w1[2] = a0.z; w1[3] = a0.w; w1[4] = a1.x; w1[5] = a1.y; w1[6] = a1.z; w1[7] = a1.w;
    w2[0] = b0.x; w2[1] = b0.y; w2[2] = b0.z; w2[3] = b0.w; w2[4] = b1.x; w2[5] = b1.y; w2[6] = b1.z; w2[7] = b1.w;
  }
  const float inv_d = 1.0f / (float)(2 * HALF);
  for (int s = blockIdx.x * ROWS + threadIdx.x / RUNS; s < g.rows; s += gridDim.x * ROWS) {
    float cv[8], sv[8];
    if (rot) {
      const int64_t to = (int64_t)s * HALF + c * 8;
      load8f(g.cos_t + to, cv);
      load8f(g.sin_t + to, sv);
    }
    // all loads of the group first, then the arithmetic and stores
    u32x4 lo[kRopeHeads], hi[kRopeHeads];
#pragma unroll
    for (int j = 0; j < kRopeHeads; ++j) {
      if (j < nh) {
        const int bh = bh0 + j, b = bh / p.H, h = bh - b * p.H;
        const bf16_t *xr = g.x + b * g.xs_b + h * g.xs_h + (int64_t)s * g.xs_s;
        lo[j] = ldg16(xr + c * 8);
        hi[j] = ldg16(xr + HALF + c * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kRopeHeads; ++j) {
      if (j < nh) {
        float x1[8], x2[8];
        unpack8(lo[j], x1);
        unpack8(hi[j], x2);
        if (nrm) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(x1[e], x1[e], fmaf(x2[e], x2[e], ss));
#pragma unroll
          for (int m = 1; m < RUNS; m <<= 1) ss += __shfl_xor(ss, m);
          const float inv = 1.0f / sqrtf(fmaf(ss, inv_d, p.eps));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x1[e] = x1[e] * inv * w1[e];
            x2[e] = x2[e] * inv * w2[e];
          }
        }
        if (rot) rotate8(x1, x2, cv, sv);
        bf16_t *yr = g.y + ((int64_t)(bh0 + j) * g.S + s) * (2 * HALF);
        *reinterpret_cast<u32x4 *>(yr + c * 8) = pack8(x1);
        *reinterpret_cast<u32x4 *>(yr + HALF + c * 8) = pack8(x2);
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnParams &p, int d, hipStream_t stream) {
  if (p.kv_seg_len > 0) {
    const int64_t nb = (int64_t)p.n_qtiles * p.H * p.B;
    if (nb <= 0) return hipSuccess;
    if (d == 128) hipLaunchKernelGGL(attn_fwd_seg_kernel<128>, dim3((unsigned)nb), dim3(NT), 0, stream, p);
    else hipLaunchKernelGGL(attn_fwd_seg_kernel<64>, dim3((unsigned)nb), dim3(NT), 0, stream, p);
    return hipGetLastError();
  }
  if (p.dyn_grid > 0) {
    if (d == 128)
      hipLaunchKernelGGL((attn_fwd_kernel<128, false, true>), dim3((unsigned)p.dyn_grid), dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<64, false, true>), dim3((unsigned)p.dyn_grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
  }
  const bool sk = p.sk_grid > 0;
  const int64_t nblocks = sk ? p.sk_grid : (int64_t)p.n_qtiles * p.H * p.B;
  if (nblocks <= 0) return hipSuccess;
  if (d == 128) {
    if (sk) hipLaunchKernelGGL((attn_fwd_kernel<128, true>), dim3((unsigned)nblocks), dim3(NT), 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false>), dim3((unsigned)nblocks), dim3(NT), 0, stream, p);
  } else {
    if (sk) hipLaunchKernelGGL((attn_fwd_kernel<64, true>), dim3((unsigned)nblocks), dim3(NT), 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false>), dim3((unsigned)nblocks), dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_rope_rotate(const RopeRotateParams &p, hipStream_t stream) {
  int rows = 0;
  for (int i = 0; i < p.n_seg; ++i) rows = p.seg[i].rows > rows ? p.seg[i].rows : rows;
  const int64_t nbh = (int64_t)p.B * p.H;
  if (p.n_seg <= 0 || rows <= 0 || nbh <= 0) return launch_zero_i32(p.zero, p.n_zero, stream);
  const int runs = p.d / 16;
  const int per_block = 256 / runs;
  int64_t bx = (rows + per_block - 1) / per_block;
  if (bx > 65535) bx = 65535;   // the kernel strides over the remaining rows
  const dim3 grid((unsigned)bx, (unsigned)p.n_seg, (unsigned)((nbh + kRopeHeads - 1) / kRopeHeads));
  if (runs == 8) hipLaunchKernelGGL(rope_rotate_kernel<8>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(rope_rotate_kernel<4>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

int attn_block_m() { return BM; }

}  // namespace dit

#if DIT_CLOCK_PROBE
// Probe build only: copy the stamps of the last launch (8 words per
// workgroup: shader clock and 100 MHz counter at loop start, then at loop
// end; 100 MHz counter at entry and after the stores; the loop's key
// tiles; one unused) to host memory; returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int dit_clock_probe_read(unsigned long long *host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(dit::g_clock_probe), sizeof(dit::g_clock_probe), 0,
                                  hipMemcpyDeviceToHost);
}
#endif
