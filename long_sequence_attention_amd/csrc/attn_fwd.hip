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
//   * Each wave owns 32 query rows. It computes S^T = K Q^T so that a lane
//     holds 16 scores of ONE query (lane % 32) per 32-key block: the row
//     max/sum are in-register reductions plus one exchange with lane ^ 32.
//   * Q stays in registers (bf16, rotated once) as the B operand of S^T.
//   * K tiles (64 keys x d) are staged row-major in LDS; V tiles are staged
//     transposed (V^T: d x 64 keys) so that the P.V contraction
//     O^T = V^T P^T reads 8 consecutive keys per lane with one 16-byte LDS read.
//   * The key order inside a 32-key block is permuted when K rows are read
//     (MFMA row m = 16a+8b+4c+j holds key 16a+8c+4b+j) so that the scores a
//     lane gets back from the S^T MFMA are exactly the 8-key runs it must feed
//     as the P^T operand of the P.V MFMA: no register shuffles for P.
//   * Softmax uses exp2 with scale*log2(e) folded into one FMA, and a lazy
//     rescale: the running max is only raised (and O, l rescaled) when a tile
//     max exceeds it by more than 8 (log2 units), so p <= 2^8 stays exact in
//     fp32/bf16 range. The result is unchanged in exact arithmetic.
//   * Pad keys: tiles past kv_valid are never visited; in the tail tile,
//     scores of keys >= kv_valid are replaced by -inf with a select (not an
//     add), and their K/V rows are staged as zeros (so 0 * NaN never occurs).
//   * Pad query rows are computed but overwritten by a select in the epilogue.
#include "common.h"

namespace dit {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup
constexpr int KPAD = 8;   // bf16 padding per K row in LDS (bank spread)
constexpr int VPAD = 8;   // bf16 padding per V^T row in LDS
constexpr float kLazyRescale = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4 ldg16(const bf16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Split-halves rotation of 8 pairs held as two packed bf16 vectors.
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

// Workgroup -> (b, h, q-tile) with consecutive tiles of a head kept on one
// XCD: the hardware deals workgroups round-robin over the 8 XCDs, so invert
// that to give each XCD a contiguous run of logical tiles (its own L2 then
// holds that head's K/V).
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnParams p) {
  constexpr int DK = D / 16;      // k-steps of the Q.K^T contraction
  constexpr int DB = D / 32;      // 32-row blocks of d in O^T
  constexpr int KS = D + KPAD;    // LDS K row stride (elements)
  constexpr int VS = BN + VPAD;   // LDS V^T row stride (elements)
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- Q operand (B of S^T): lane holds query qrow, d = dk*16 + hf*8 + e.
  const int qrow = qt * BM + wave * 32 + l32;
  bf16x8 qop[DK];
  {
    u32x4 raw[DK];
    const bool in_q = qrow < p.s_q;
    const bf16_t *qr = qbase + (int64_t)(in_q ? qrow : 0) * p.qs_s;
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      raw[dk] = in_q ? ldg16(qr + dk * 16 + hf * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (p.cos_q != nullptr) {
      // pair (i, i + D/2) lives in (dk, dk + DK/2) of the same lane
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

  float m_run = -INFINITY;   // running max, log2 units (already scaled)
  float l_run = 0.f;         // this lane's partial row sum (16 of 32 keys per block)
  f32x16 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};

  // K row this lane reads as MFMA row m = l32 (see the key permutation above)
  const int kperm = (l32 & 16) + ((l32 & 4) << 1) + ((l32 & 8) >> 1) + (l32 & 3);

  const int kv_valid = p.kv_valid;
  const int n_tiles = (kv_valid + BN - 1) / BN;
  for (int t = 0; t < n_tiles; ++t) {
    const int j0 = t * BN;
    __syncthreads();
    // ---- stage K tile, row-major, rows >= kv_valid as zeros
    constexpr int CPR = D / 8;               // 16-byte chunks per row
#pragma unroll
    for (int c = tid; c < BN * CPR; c += NT) {
      const int r = c / CPR, c8 = c % CPR;
      const int key = j0 + r;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (key < kv_valid) val = ldg16(kbase + (int64_t)key * p.ks_s + c8 * 8);
      *reinterpret_cast<u32x4 *>(Ks + r * KS + c8 * 8) = val;
    }
    // ---- stage V tile transposed: units of 4 keys x 8 channels
#pragma unroll
    for (int u = tid; u < (BN / 4) * CPR; u += NT) {
      const int kg = u / CPR, c8 = u % CPR;
      u32x4 rw[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = j0 + kg * 4 + rr;
        rw[rr] = (key < kv_valid) ? ldg16(vbase + (int64_t)key * p.vs_s + c8 * 8) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 ev = {(rw[0][w] & 0xffffu) | (rw[1][w] << 16), (rw[2][w] & 0xffffu) | (rw[3][w] << 16)};
        const u32x2 od = {(rw[0][w] >> 16) | (rw[1][w] & 0xffff0000u), (rw[2][w] >> 16) | (rw[3][w] & 0xffff0000u)};
        *reinterpret_cast<u32x2 *>(Vt + (c8 * 8 + 2 * w) * VS + kg * 4) = ev;
        *reinterpret_cast<u32x2 *>(Vt + (c8 * 8 + 2 * w + 1) * VS + kg * 4) = od;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sacc[blk] = f32x16{};
      const bf16_t *krow = Ks + (blk * 32 + kperm) * KS + hf * 8;
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + dk * 16);
        sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[dk], sacc[blk], 0, 0, 0);
      }
    }

    // ---- tail mask: lane (hf), reg r of block blk holds key
    //      j0 + blk*32 + 16*(r>>3) + 8*hf + (r&7)
    if (j0 + BN > kv_valid) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + blk * 32 + ((r & 8) << 1) + 8 * hf + (r & 7);
          sacc[blk][r] = (key < kv_valid) ? sacc[blk][r] : -INFINITY;
        }
      }
    }

    // ---- online softmax (exp2 form, lazy rescale)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mts = mx * p.scale_log2;
    const bool upd = mts > m_run + kLazyRescale;
    if (__any(upd)) {
      const float m_new = upd ? mts : m_run;
      const float alpha = (m_new == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
    const float neg_m = -m_run;
    bf16x8 pop[2][2];
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[blk][8 * a + e], p.scale_log2, neg_m));
          psum += pv[e];
        }
        pop[blk][a] = __builtin_convertvector(pv, bf16x8);
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16_t *vrow = Vt + (db * 32 + l32) * VS + hf * 8;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const bf16x8 vv = *reinterpret_cast<const bf16x8 *>(vrow + blk * 32 + a * 16);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pop[blk][a], acc_o[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O = acc / l; LSE = (m + log2 l) ln 2; pad rows by select
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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

// K rotation pre-pass: y = rope(x) for rows < valid, dense [B, H, S, d] bf16.
// One thread per (row, run of 8 pairs).
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
