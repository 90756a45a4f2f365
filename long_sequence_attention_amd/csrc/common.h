// Shared device helpers and launcher declarations for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;  // bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 -> fp32 is exact: the pattern is the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Eight bf16 from one 16-byte word group -> fp32, and back (round to nearest even).
__device__ __forceinline__ void unpack8(const u32x4 &v, float *x) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = bf16_lo(v[w]);
    x[2 * w + 1] = bf16_hi(v[w]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float *x) {
  return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

// Split-halves rotation of 8 channel pairs in fp32: x1 holds channels
// i..i+7 of the first half, x2 the partners d/2 later. Every kernel that
// rotates uses this one routine, so they all round alike.
__device__ __forceinline__ void rotate8(float *x1, float *x2, const float *cv, const float *sv) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y1 = fmaf(x1[e], cv[e], -x2[e] * sv[e]);
    const float y2 = fmaf(x2[e], cv[e], x1[e] * sv[e]);
    x1[e] = y1;
    x2[e] = y2;
  }
}

// Eight consecutive fp32 table entries (32-byte aligned run).
__device__ __forceinline__ void load8f(const float *t, float *x) {
  const float4 a = *reinterpret_cast<const float4 *>(t);
  const float4 b = *reinterpret_cast<const float4 *>(t + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Attention tiling shared by the kernels and the host planning code: a
// workgroup of kAttnWaves waves owns kAttnBlockM = 32 * kAttnWaves query
// rows of one head and walks the keys in tiles of kAttnBlockN rows.
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnBlockM = 32 * kAttnWaves;
constexpr int kAttnBlockN = 64;

// Fixed-m softmax: per-(b, h) key statistics over the real keys and the
// per-row bound m_i = c2 * (q_i . kbar + |q_i| R), R = max_j |k_j - kbar|
// (log2 units), plus a per-q-tile flag: 1 when every real row of the tile
// has a bound spread 2 c2 |q_i| R small enough for the fixed maximum.
constexpr int kStatRows = 256;   // key rows per statistics chunk
struct FixedMParams {
  const bf16_t *q, *k;
  int64_t qs_b, qs_h, qs_s, ks_b, ks_h, ks_s;
  int32_t B, H, d, s_q, s_kv, q_valid, kv_valid, q_seg_len, kv_seg_len;
  int32_t n_chunks, n_real, n_qtiles;
  float c2;
  float *part;   // [B*H][n_chunks][d] partial key sums
  float *kbar;   // [B*H][d] key mean
  float *r2;     // [B*H][n_chunks] max |k_j - kbar|^2 of each chunk
  float *m;      // [B*H][s_q] row bounds
  int32_t *ok;   // [B*H][n_qtiles] fixed-m usable for the q-tile
};

// Parameters of the attention forward kernel (passed by value).
struct AttnParams {
  const bf16_t *q, *k, *v;
  void *o;
  float *lse;
  int64_t qs_b, qs_h, qs_s;
  int64_t ks_b, ks_h, ks_s;
  int64_t vs_b, vs_h, vs_s;
  int64_t os_b, os_h, os_s;
  int32_t B, H, s_q, s_kv, q_valid, kv_valid;
  // segments padded at their own tails (0 = one segment): q_valid / kv_valid
  // then count the real rows of each segment
  int32_t q_seg_len, kv_seg_len, n_kv_seg;
  int32_t o_f32;
  int32_t n_qtiles;
  float scale_log2;  // sm_scale * log2(e)
  // split schedule (sk_grid > 0 workgroups): sk_main main workgroups (one
  // per q-tile, keys [0, sk_kc)) and sk_grid - sk_main helpers splitting the
  // remaining key tails Stream-K style (sk_main = sk_kc = 0: plain Stream-K
  // over every unit); the pieces of a q-tile meet in the workspace below
  int32_t sk_grid, sk_main, sk_kc;
  float *sk_part_o;  // [2 sk_grid slots][kAttnThreads][d/2] partial O / l, fp32
  float *sk_part_l;  // [2 sk_grid slots][kAttnBlockM rows] partial LSE, log2 units
  int32_t *sk_count; // [q-tiles] arrival counters, zero on entry (left zero on exit);
                     // dynamic placement: [0..7] next tile of each XCD queue, [8] tiles taken
  // dynamic placement (dyn_grid > 0 workgroups, more than the q-tiles; the
  // first dyn_static take their q-tile by index, the rest through the
  // sk_count queue counters; 0 = off)
  int32_t dyn_grid, dyn_static;
  // fixed-m softmax (fm_m != nullptr): row bounds [B*H][s_q] and per-q-tile
  // flags [B*H][n_qtiles] from launch_fixed_m
  const float *fm_m;
  const int32_t *fm_ok;
};

// One tensor of the pre-pass: rows [0, rows) of x ((b, h, s) strides in
// elements) RMS-normalised with the fp32 [d] weights norm_w (when non-NULL),
// rotated with the fp32 [>= rows, d/2] tables cos_t / sin_t (when non-NULL)
// and written to the dense [B, H, S, d] buffer y.
struct RopeSeg {
  const bf16_t *x;
  bf16_t *y;
  const float *cos_t, *sin_t;
  const float *norm_w;
  int64_t xs_b, xs_h, xs_s;
  int32_t S, rows;
};

// Parameters of the Q / K pre-pass (one launch for both tensors). zero /
// n_zero: int32 words the launch also clears (the Stream-K arrival
// counters of the attention launch that follows), or NULL / 0.
struct RopeRotateParams {
  RopeSeg seg[2];
  int32_t n_seg, B, H, d;
  float eps;   // RMSNorm epsilon
  int32_t *zero;
  int32_t n_zero;
};

// Tail pad of fused token rows with the rotation on the way: in [B, s_valid,
// T, H, d] -> out [B, s_pad, T, H, d] (dense, token-major), tensors t < n_rot
// of every real row rotated with the fp32 [>= s_valid, d/2] tables, the
// others copied, rows >= s_valid zero.
struct PadRopeParams {
  const bf16_t *in;
  bf16_t *out;
  const float *cos_t, *sin_t;
  int32_t s_valid, s_pad, T, H, n_rot;
};

constexpr int kMaxMergeParts = 16;
struct MergeParams {
  const void *o_parts[kMaxMergeParts];
  const float *lse_parts[kMaxMergeParts];
  void *o_out;
  float *lse_out;
  int32_t n_parts, part_f32, out_f32, rows, S, d, q_valid;
};

constexpr int kMaxPairs = 128;
struct TableParams {
  double freq[kMaxPairs];
  uint8_t axis[kMaxPairs];
  const int32_t *pos;
  float *cos_out, *sin_out;
  int32_t S, n_axes, half_d;
};

// Launchers (host side, defined next to their kernels). Return hipError_t.
hipError_t launch_attn_fwd(const AttnParams &p, int d, hipStream_t stream);
hipError_t launch_fixed_m(const FixedMParams &p, hipStream_t stream);
hipError_t launch_zero_i32(int32_t *p, int64_t n, hipStream_t stream);
hipError_t launch_rope_rotate(const RopeRotateParams &p, hipStream_t stream);
hipError_t launch_lse_merge(const MergeParams &p, hipStream_t stream);
hipError_t launch_rope_tables(const TableParams &p, hipStream_t stream);
hipError_t launch_row_copy(const void *in, void *out, int B, int s_in, int s_out, int n_copy,
                           int64_t row_bytes, hipStream_t stream);
hipError_t launch_pad_rope(const PadRopeParams &p, int B, int d, hipStream_t stream);

}  // namespace dit
