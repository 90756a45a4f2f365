// HBM-bound passes of the DiT attention path on gfx950:
//   * RoPE cos/sin tables from integer positions (Difflet PR #153, FLUX
//     split-RoPE commit: tables built once per forward, split-halves order);
//   * tail pad / unpad of token rows (Difflet PR #153 Wan padding commit;
//     maxdiffusion PR #491 lane padding), and the pad of fused Q/K/V rows
//     with the split-halves rotation of Q and K applied on the way;
//   * the LSE merge of per-key-shard partial results (mstar PR #376,
//     attention_over_sharded_keys).
// Each is a streaming pass: 16-byte vector loads/stores, consecutive lanes on
// consecutive addresses, no LDS.
#include "common.h"

namespace dit {

namespace {

// One thread per table entry (s, pair j): angle = pos[s, axis(j)] * freq[j]
// evaluated in fp64, cos/sin in fp64, rounded once to fp32.
// (S * d/2 < 2^31 is checked by the caller, so the index math is 32-bit.)
__global__ __launch_bounds__(256) void rope_tables_kernel(TableParams p) {
  const int total = p.S * p.half_d;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
    const int s = t / p.half_d;
    const int j = t - s * p.half_d;
    const double ang = (double)p.pos[(int64_t)s * p.n_axes + p.axis[j]] * p.freq[j];
    double sn, cs;
    sincos(ang, &sn, &cs);
    p.cos_out[t] = (float)cs;
    p.sin_out[t] = (float)sn;
  }
}

// The same tables, PER consecutive pairs of one row per thread (used when
// half_d is a multiple of PER and the outputs are 16-byte aligned): the PER
// angles are independent, so their fp64 cos/sin overlap, and each output
// leaves as one PER x 4-byte store. Same arithmetic per entry, same bits.
template <int PER>
__global__ __launch_bounds__(256) void rope_tables_vec_kernel(TableParams p) {
  typedef float fvec __attribute__((ext_vector_type(PER)));
  const int per_row = p.half_d / PER;
  const int total = p.S * per_row;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
    const int s = t / per_row;
    const int j0 = (t - s * per_row) * PER;
    const int32_t *ps = p.pos + (int64_t)s * p.n_axes;
    fvec cv, sv;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const double ang = (double)ps[p.axis[j0 + e]] * p.freq[j0 + e];
      double sn, cs;
      sincos(ang, &sn, &cs);
      cv[e] = (float)cs;
      sv[e] = (float)sn;
    }
    *reinterpret_cast<fvec *>(p.cos_out + (int64_t)s * p.half_d + j0) = cv;
    *reinterpret_cast<fvec *>(p.sin_out + (int64_t)s * p.half_d + j0) = sv;
  }
}

// Tail pad / unpad of one batch (blockIdx.y): rows 0..n_copy-1 of both
// sides are one contiguous run, so out[i] = in[i] for i < n_copy granules
// and out[i] = 0 up to n_total. V is the copy granule (16, 4 or 1 bytes),
// chosen from the row size and alignment. UNROLL granules per thread are in
// flight, a grid stride apart, so consecutive lanes stay on consecutive
// addresses. STREAM: the source is read with non-temporal loads (it is dead
// after the copy; the result is stored normally, so the next kernel can
// still find it in the caches).
template <typename V, int UNROLL, bool STREAM>
__global__ __launch_bounds__(256) void row_copy_kernel(const V *__restrict__ in, V *__restrict__ out,
                                                      int64_t in_batch, int64_t out_batch, int64_t n_copy,
                                                      int64_t n_total) {
  const V *src = in + (int64_t)blockIdx.y * in_batch;
  V *dst = out + (int64_t)blockIdx.y * out_batch;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < n_total; i0 += stride * UNROLL) {
    V v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = (i < n_copy) ? (STREAM ? __builtin_nontemporal_load(src + i) : src[i]) : V{};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n_total) dst[i] = v[u];
    }
  }
}

template <int PER>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParams p) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= p.rows) return;
  const int sub = threadIdx.x & 31;
  const int i = (int)(row % p.S);
  const int64_t off = row * p.d + sub * PER;
  // every part's LSE and O chunk is requested before any arithmetic, so a
  // thread keeps n_parts loads in flight (the partials are read once:
  // non-temporal loads)
  float L[kMaxMergeParts];
  float val[kMaxMergeParts][PER];
#pragma unroll
  for (int k = 0; k < kMaxMergeParts; ++k) {
    if (k < p.n_parts) {
      L[k] = p.lse_parts[k][row];
      if (p.part_f32) {
        const float *src = reinterpret_cast<const float *>(p.o_parts[k]) + off;
#pragma unroll
        for (int e = 0; e < PER; ++e) val[k][e] = __builtin_nontemporal_load(src + e);
      } else {
        const bf16_t *src = reinterpret_cast<const bf16_t *>(p.o_parts[k]) + off;
#pragma unroll
        for (int e = 0; e < PER; ++e) val[k][e] = __uint_as_float((uint32_t)__builtin_nontemporal_load(src + e) << 16);
      }
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxMergeParts; ++k)
    if (k < p.n_parts) M = fmaxf(M, L[k]);
  const bool empty = (M == -INFINITY) || (i >= p.q_valid);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (!empty) {
#pragma unroll
    for (int k = 0; k < kMaxMergeParts; ++k) {
      if (k < p.n_parts) {
        const float w = expf(L[k] - M);
        wsum += w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, val[k][e], acc[e]);
      }
    }
  }
  const float inv = empty ? 0.f : 1.0f / wsum;
  if (p.out_f32) {
    float *dst = reinterpret_cast<float *>(p.o_out) + off;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = empty ? 0.f : acc[e] * inv;
  } else {
    bf16_t *dst = reinterpret_cast<bf16_t *>(p.o_out) + off;
#pragma unroll
    for (int e = 0; e < PER; e += 2) {
      const uint32_t w = pack_bf16x2(empty ? 0.f : acc[e] * inv, empty ? 0.f : acc[e + 1] * inv);
      *reinterpret_cast<uint32_t *>(dst + e) = w;
    }
  }
  if (p.lse_out != nullptr && sub == 0) p.lse_out[row] = empty ? -INFINITY : M + logf(wsum);
}

// Tail pad of fused token rows with the split-halves rotation applied on the
// way: one pass over Q, K and V instead of a pad copy followed by a rotation
// pass over Q and K (the pages fuse the rotation into neighbouring work). A
// task is one 8-channel run of one head vector and its partner run d/2 later
// (2 x 16 bytes); consecutive lanes take consecutive runs, so a wave reads and
// writes whole rows. Head vectors of the first n_rot tensors of a real row are
// rotated with that row's tables by rotate8, the routine of the attention
// pre-pass, so the two paths give the same bits; the others are copied; pad
// rows are written as zeros. STREAM: the source rows are read with
// non-temporal loads (copies larger than the MALL, as in row_copy_kernel).
// (T * H * RUNS * s_pad < 2^31 is checked by the caller, so the task index
// is 32-bit.)
template <int RUNS, bool STREAM>
__global__ __launch_bounds__(256) void pad_rope_kernel(PadRopeParams p) {
  constexpr int HALF = RUNS * 8;
  const uint32_t vecs = (uint32_t)(p.T * p.H);
  const uint32_t per_row = vecs * RUNS;
  const uint32_t total = per_row * (uint32_t)p.s_pad;
  const uint32_t n_rot_vecs = (uint32_t)(p.n_rot * p.H);
  const int64_t row_elems = (int64_t)vecs * (2 * HALF);
  const bf16_t *src = p.in + (int64_t)blockIdx.y * p.s_valid * row_elems;
  bf16_t *dst = p.out + (int64_t)blockIdx.y * p.s_pad * row_elems;
  for (uint32_t g = blockIdx.x * 256u + threadIdx.x; g < total; g += gridDim.x * 256u) {
    const uint32_t s = g / per_row;
    const uint32_t r = g - s * per_row;
    const uint32_t vec = r / RUNS, c = r % RUNS;
    const int64_t off = (int64_t)s * row_elems + (int64_t)vec * (2 * HALF) + c * 8;
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (s < (uint32_t)p.s_valid) {
      const u32x4 *a = reinterpret_cast<const u32x4 *>(src + off);
      const u32x4 *b = reinterpret_cast<const u32x4 *>(src + off + HALF);
      lo = STREAM ? __builtin_nontemporal_load(a) : *a;
      hi = STREAM ? __builtin_nontemporal_load(b) : *b;
      if (vec < n_rot_vecs) {
        float cv[8], sv[8], x1[8], x2[8];
        load8f(p.cos_t + (int64_t)s * HALF + c * 8, cv);
        load8f(p.sin_t + (int64_t)s * HALF + c * 8, sv);
        unpack8(lo, x1);
        unpack8(hi, x2);
        rotate8(x1, x2, cv, sv);
        lo = pack8(x1);
        hi = pack8(x2);
      }
    }
    *reinterpret_cast<u32x4 *>(dst + off) = lo;
    *reinterpret_cast<u32x4 *>(dst + off + HALF) = hi;
  }
}

int grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return (int)(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_rope_tables(const TableParams &p, hipStream_t stream) {
  const int64_t total = (int64_t)p.S * p.half_d;
  if (total <= 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(p.cos_out) | reinterpret_cast<uintptr_t>(p.sin_out);
  if (p.half_d % 4 == 0 && al % 16 == 0)
    hipLaunchKernelGGL(rope_tables_vec_kernel<4>, dim3(grid_for(total / 4)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rope_tables_kernel, dim3(grid_for(total)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Copies that fit the 256 MB MALL (the Wan 480p / FLUX token tensors) run
// four granules per thread on at most 4096 blocks; larger ones stream one
// granule per thread on up to 32768 blocks with non-temporal source loads
// (measured on MI355X: 6.8 TB/s against 4.8 TB/s for the small-copy form
// on a 387 MB pad, while the small-copy form makes the Wan 480p step, whose
// pad and unpad move 24-73 MB each, about 1 us faster).
template <typename V>
static void launch_copy_v(const void *in, void *out, int B, int s_in, int s_out, int n_copy, int64_t row_bytes,
                          hipStream_t stream) {
  const int64_t rv = row_bytes / (int64_t)sizeof(V);
  const int64_t n_total = (int64_t)s_out * rv;
  const bool large = (int64_t)B * n_total * (int64_t)sizeof(V) * 2 > (128LL << 20);
  const dim3 blk(256);
  const V *src = static_cast<const V *>(in);
  V *dst = static_cast<V *>(out);
  if (large) {
    int64_t blocks = (n_total + 255) / 256;
    if (blocks > 32768) blocks = 32768;
    hipLaunchKernelGGL((row_copy_kernel<V, 1, true>), dim3((unsigned)blocks, (unsigned)B), blk, 0, stream, src, dst,
                       (int64_t)s_in * rv, n_total, (int64_t)n_copy * rv, n_total);
  } else {
    int64_t blocks = (n_total + 1023) / 1024;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL((row_copy_kernel<V, 4, false>), dim3((unsigned)blocks, (unsigned)B), blk, 0, stream, src,
                       dst, (int64_t)s_in * rv, n_total, (int64_t)n_copy * rv, n_total);
  }
}

hipError_t launch_row_copy(const void *in, void *out, int B, int s_in, int s_out, int n_copy,
                           int64_t row_bytes, hipStream_t stream) {
  if ((int64_t)B * s_out * row_bytes == 0) return hipSuccess;
  const uintptr_t a = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out);
  if (row_bytes % 16 == 0 && a % 16 == 0) launch_copy_v<u32x4>(in, out, B, s_in, s_out, n_copy, row_bytes, stream);
  else if (row_bytes % 4 == 0 && a % 4 == 0) launch_copy_v<uint32_t>(in, out, B, s_in, s_out, n_copy, row_bytes, stream);
  else launch_copy_v<uint8_t>(in, out, B, s_in, s_out, n_copy, row_bytes, stream);
  return hipGetLastError();
}

hipError_t launch_pad_rope(const PadRopeParams &p, int B, int d, hipStream_t stream) {
  const int64_t total = (int64_t)p.T * p.H * (d / 16) * p.s_pad;
  if (total <= 0 || B <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;   // the kernel strides over the rest
  const dim3 grid((unsigned)blocks, (unsigned)B);
  // the same size rule as the row copies: reads and writes together beyond
  // 128 MB take the non-temporal source loads
  const bool large = (int64_t)B * total * 32 * 2 > (128LL << 20);
  if (d == 128) {
    if (large) hipLaunchKernelGGL((pad_rope_kernel<8, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((pad_rope_kernel<8, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (large) hipLaunchKernelGGL((pad_rope_kernel<4, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((pad_rope_kernel<4, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t blocks = ((int64_t)p.rows + 7) / 8;
  if (p.d == 128) {
    hipLaunchKernelGGL(lse_merge_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dit
