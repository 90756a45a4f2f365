// Statistics for the fixed-m softmax (maxdiffusion PR #491: fixed-m metadata
// from norm reductions and the key mean over the real rows, with blocks whose
// bound is too loose sent to the online-softmax path). The bound used is
//   m_i = scale * (q_i . kbar + |q_i| * max_j |k_j - kbar|)
// (Cauchy-Schwarz on q_i . (k_j - kbar)), over the real keys j only; it is
// computed from the same bf16 Q and K the attention kernel multiplies.
// Every reduction runs in a fixed order, so the bounds (and the attention
// results that use them) are the same bits on every call.
#include "common.h"

namespace dit {

namespace {

__device__ __forceinline__ bool key_is_real(const FixedMParams &p, int j) {
  return j < p.s_kv && (p.kv_seg_len > 0 ? j % p.kv_seg_len < p.kv_valid : j < p.kv_valid);
}

__device__ __forceinline__ bool query_row_is_real(const FixedMParams &p, int i) {
  return i < p.s_q && (p.q_seg_len > 0 ? i % p.q_seg_len < p.q_valid : i < p.q_valid);
}

// Partial key sums of chunk blockIdx.x of head blockIdx.y: TPR = D/8 lanes
// per row (8 channels each), 256/TPR rows per pass; every pass's load is
// issued before any is used, then the row groups are added in a fixed order
// through LDS.
template <int D>
__global__ __launch_bounds__(256) void key_sum_kernel(FixedMParams p) {
  constexpr int TPR = D / 8, RPB = 256 / TPR, RPT = kStatRows / RPB;
  __shared__ float red[256 * 8];
  const int lc = threadIdx.x % TPR, rs = threadIdx.x / TPR;
  const int bh = blockIdx.y, b = bh / p.H, h = bh - b * p.H;
  const bf16_t *kh = p.k + b * p.ks_b + h * p.ks_h;
  u32x4 raw[RPT];
#pragma unroll
  for (int t = 0; t < RPT; ++t) {
    const int j = blockIdx.x * kStatRows + t * RPB + rs;
    raw[t] = key_is_real(p, j) ? *reinterpret_cast<const u32x4 *>(kh + (int64_t)j * p.ks_s + lc * 8)
                               : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < RPT; ++t) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += bf16_lo(raw[t][w]);
      acc[2 * w + 1] += bf16_hi(raw[t][w]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[threadIdx.x * 8 + e] = acc[e];
  __syncthreads();
  for (int ch = threadIdx.x; ch < D; ch += 256) {
    float s = 0.f;
    for (int g = 0; g < RPB; ++g) s += red[(g * TPR + ch / 8) * 8 + ch % 8];
    p.part[((int64_t)bh * p.n_chunks + blockIdx.x) * D + ch] = s;
  }
}

// Key mean of head blockIdx.x: the chunks' partial sums in chunk order, with
// eight partials in flight per thread.
__global__ __launch_bounds__(256) void key_mean_kernel(FixedMParams p) {
  const int bh = blockIdx.x;
  for (int ch = threadIdx.x; ch < p.d; ch += 256) {
    const float *src = p.part + (int64_t)bh * p.n_chunks * p.d + ch;
    float s = 0.f;
    int c = 0;
    for (; c + 8 <= p.n_chunks; c += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = src[(int64_t)(c + u) * p.d];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    for (; c < p.n_chunks; ++c) s += src[(int64_t)c * p.d];
    p.kbar[(int64_t)bh * p.d + ch] = s / (float)p.n_real;
  }
}

// Largest |x - kbar|^2 over a thread's rows (RPT rows a pass apart, TPR lanes
// per row, all loads issued first); rows that are not real give 0.
template <int D, int RPT, class F>
__device__ __forceinline__ void spread_rows(const bf16_t *base, int64_t stride, int row0, int rs, int lc,
                                            const float *kb, F is_real, float *qq_out, float *qk_out,
                                            bool *real_out) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  u32x4 raw[RPT];
  bool real[RPT];
#pragma unroll
  for (int t = 0; t < RPT; ++t) {
    const int j = row0 + t * RPB + rs;
    real[t] = is_real(j);
    raw[t] = real[t] ? *reinterpret_cast<const u32x4 *>(base + (int64_t)j * stride + lc * 8) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int t = 0; t < RPT; ++t) {
    float x[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = bf16_lo(raw[t][w]);
      x[2 * w + 1] = bf16_hi(raw[t][w]);
    }
    float a = 0.f, c = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a = fmaf(x[e] - kb[e], x[e] - kb[e], a);   // |x - kbar|^2 part (keys)
      c = fmaf(x[e], x[e], c);                   // |x|^2 part (queries)
    }
    const float kbx = [&] {
      float r = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) r = fmaf(x[e], kb[e], r);
      return r;
    }();
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) {
      a += __shfl_xor(a, m);
      c += __shfl_xor(c, m);
    }
    float k2 = kbx;
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) k2 += __shfl_xor(k2, m);
    qq_out[t] = qk_out == nullptr ? a : c;
    if (qk_out != nullptr) qk_out[t] = k2;
    real_out[t] = real[t];
  }
}

// max |k_j - kbar|^2 over the real rows of chunk blockIdx.x of head
// blockIdx.y.
template <int D>
__global__ __launch_bounds__(256) void key_spread_kernel(FixedMParams p) {
  constexpr int TPR = D / 8, RPB = 256 / TPR, RPT = kStatRows / RPB;
  __shared__ float red[256];
  const int lc = threadIdx.x % TPR, rs = threadIdx.x / TPR;
  const int bh = blockIdx.y, b = bh / p.H, h = bh - b * p.H;
  float kb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) kb[e] = p.kbar[(int64_t)bh * D + lc * 8 + e];
  float d2[RPT];
  bool real[RPT];
  spread_rows<D, RPT>(p.k + b * p.ks_b + h * p.ks_h, p.ks_s, blockIdx.x * kStatRows, rs, lc, kb,
                      [&](int j) { return key_is_real(p, j); }, d2, nullptr, real);
  float best = 0.f;
#pragma unroll
  for (int t = 0; t < RPT; ++t)
    if (real[t]) best = fmaxf(best, d2[t]);
  red[threadIdx.x] = best;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) p.r2[(int64_t)bh * p.n_chunks + blockIdx.x] = red[0];
}

// Row bounds and the q-tile flag of q-tile blockIdx.x of head blockIdx.y.
// The spread 2 c2 |q_i| R bounds how far below m_i any score of row i can
// fall; above kMaxSpread (log2 units) the probability of the row's best key
// could leave the normal fp32 / bf16 range, so the q-tile keeps the online
// softmax.
constexpr float kMaxSpread = 96.0f;

template <int D>
__global__ __launch_bounds__(256) void query_bound_kernel(FixedMParams p) {
  constexpr int TPR = D / 8, RPB = 256 / TPR, RPT = kAttnBlockM / RPB;
  __shared__ float red[256];
  __shared__ int bad_sh;
  const int lc = threadIdx.x % TPR, rs = threadIdx.x / TPR;
  const int bh = blockIdx.y, b = bh / p.H, h = bh - b * p.H;
  // R^2: the chunk maxima, strided over the block, then a tree in LDS
  float mx = 0.f;
  for (int c = threadIdx.x; c < p.n_chunks; c += 256) mx = fmaxf(mx, p.r2[(int64_t)bh * p.n_chunks + c]);
  red[threadIdx.x] = mx;
  if (threadIdx.x == 0) bad_sh = 0;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float R = sqrtf(red[0]);
  float kb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) kb[e] = p.kbar[(int64_t)bh * D + lc * 8 + e];
  float qq[RPT], qk[RPT];
  bool in_q[RPT];
  const int row0 = blockIdx.x * kAttnBlockM;
  spread_rows<D, RPT>(p.q + b * p.qs_b + h * p.qs_h, p.qs_s, row0, rs, lc, kb,
                      [&](int i) { return i < p.s_q; }, qq, qk, in_q);
  int bad = 0;
#pragma unroll
  for (int t = 0; t < RPT; ++t) {
    const int i = row0 + t * RPB + rs;
    const float qn = sqrtf(qq[t]);
    if (in_q[t] && lc == 0) p.m[(int64_t)bh * p.s_q + i] = p.c2 * fmaf(qn, R, qk[t]);
    // a real row whose spread is too wide (or not finite) sends the q-tile
    // to the online softmax
    if (query_row_is_real(p, i) && !(2.0f * p.c2 * qn * R <= kMaxSpread)) bad = 1;
  }
  if (bad) bad_sh = 1;   // every writer stores the same value
  __syncthreads();
  if (threadIdx.x == 0) p.ok[(int64_t)bh * p.n_qtiles + blockIdx.x] = bad_sh ? 0 : 1;
}

}  // namespace

hipError_t launch_fixed_m(const FixedMParams &p, hipStream_t stream) {
  const unsigned bh = (unsigned)(p.B * p.H);
  if (bh == 0 || p.n_qtiles <= 0) return hipSuccess;
  const dim3 blk(256), gk((unsigned)p.n_chunks, bh), gq((unsigned)p.n_qtiles, bh);
  if (p.d == 128) {
    hipLaunchKernelGGL(key_sum_kernel<128>, gk, blk, 0, stream, p);
    hipLaunchKernelGGL(key_mean_kernel, dim3(bh), blk, 0, stream, p);
    hipLaunchKernelGGL(key_spread_kernel<128>, gk, blk, 0, stream, p);
    hipLaunchKernelGGL(query_bound_kernel<128>, gq, blk, 0, stream, p);
  } else {
    hipLaunchKernelGGL(key_sum_kernel<64>, gk, blk, 0, stream, p);
    hipLaunchKernelGGL(key_mean_kernel, dim3(bh), blk, 0, stream, p);
    hipLaunchKernelGGL(key_spread_kernel<64>, gk, blk, 0, stream, p);
    hipLaunchKernelGGL(query_bound_kernel<64>, gq, blk, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dit
