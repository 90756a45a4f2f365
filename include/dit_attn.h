/*
 * dit_attn.h -- C ABI of the MI355X (gfx950) DiT self-attention library.
 *
 * One GPU's part of full-sequence self-attention inside a video/image
 * diffusion transformer after a Ulysses head split: all S tokens, a share of
 * the heads. The calls follow the pages' problem statement:
 *   - split-halves RoPE tables and rotation (Difflet PR #153 "TPU sequence
 *     parallelism ...": FLUX split-RoPE commit and the Wan padding + split
 *     RoPE commit);
 *   - attention forward returning O and the natural-log log-sum-exp per query
 *     row, with tail-pad keys dropped exactly (mstar PR #376, ragged attention
 *     "return_lse"; maxdiffusion PR #491, the ragged KV tail carries the real
 *     length);
 *   - the merge of per-key-shard (O, LSE) pairs (mstar PR #376,
 *     attention_over_sharded_keys);
 *   - tail pad / unpad of token rows (Difflet PR #153 Wan padding commit;
 *     maxdiffusion PR #491 lane padding).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers unless stated otherwise. The
 *     caller owns every buffer; the library never allocates or frees device
 *     memory and keeps no state between calls.
 *   - bf16 data is passed as 16-bit storage (uint16_t bit patterns).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream` and returns without
 *     synchronising. Outputs must not alias inputs.
 *   - Arguments are validated before any HIP call. A bad argument returns
 *     DIT_ERR_INVALID; a valid request the kernels do not cover returns
 *     DIT_ERR_UNSUPPORTED (there is no silent fallback); a failed launch
 *     returns DIT_ERR_HIP. dit_last_error() then describes the failure.
 *     Nothing throws across the ABI.
 */
#ifndef DIT_ATTN_H_
#define DIT_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define DIT_API __attribute__((visibility("default")))
#else
#define DIT_API
#endif

typedef enum {
  DIT_OK = 0,
  DIT_ERR_INVALID = -1,
  DIT_ERR_UNSUPPORTED = -2,
  DIT_ERR_HIP = -3
} dit_status;

typedef enum { DIT_BF16 = 0, DIT_F32 = 1 } dit_dtype;

/* How dit_attn_fwd spreads work over the GPU (results agree to rounding;
 * each schedule is bit-reproducible from call to call):
 * PER_QTILE runs one workgroup per 256-row query tile over all keys.
 * BALANCED (Stream-K) runs one workgroup per compute unit: the launch's
 * (query tile, 64-key tile) units, query-tile major, are cut into equal
 * contiguous ranges, one per workgroup, so every compute unit gets the same
 * work; a query tile whose keys span two or three ranges is finished in
 * pieces: each piece writes fp32 partial results to the workspace and the
 * last piece of the tile to arrive merges them in key order (no workgroup
 * waits for another). It covers one-segment, online-softmax calls with at
 * least two key tiles; other calls run PER_QTILE.
 * With fewer query tiles than compute units, BALANCED keeps one "main"
 * workgroup per query tile on the keys' head (all in step, so each K/V tile
 * is read while it is in L2) and lets the spare compute units split the
 * remaining key tails. AUTO never takes BALANCED: on MI355X the split
 * measured slower on every shape tried. Its loop over pieces leaves the
 * kernel short of registers (spilled scalar and vector registers), so its
 * key loop issues MFMAs about 30% slower than PER_QTILE's; and the chip is
 * power-limited, so even at PER_QTILE's rate the clock falls as the spare
 * compute units join, which leaves less to gain than the partial results'
 * store and merge cost.
 * DYNAMIC keeps one workgroup per query tile but lets the workgroups take
 * their tiles at run time: the tiles, in (b, h, tile) order, form eight
 * queues (those PER_QTILE places on each of the eight XCDs), a workgroup
 * takes the next tile of its own XCD's queue, else of the others, through
 * device-scope counters in the workspace, and the grid has a sixteenth more
 * workgroups than tiles (the spares exit when every queue is empty). The
 * XCDs of an MI355X each run at their own clock under the power limit, so
 * with several waves of tiles the XCDs that get through their queue first
 * take over tiles the slower ones have not started. Each tile is computed
 * exactly as under PER_QTILE, so the results are the same bits. Calls with
 * key segments run PER_QTILE. AUTO resolves to DYNAMIC from four waves of
 * query tiles (four per compute unit), else to PER_QTILE: with fewer waves
 * the counters' contention when a wave starts costs more than the
 * rebalancing saves. */
typedef enum {
  DIT_SCHED_AUTO = 0,
  DIT_SCHED_PER_QTILE = 1,
  DIT_SCHED_BALANCED = 2,
  DIT_SCHED_DYNAMIC = 3
} dit_schedule;

/*
 * Attention forward descriptor.
 *
 * Q, K, V, O are logically [B, H, S, d] with d contiguous. Element strides
 * for (b, h, s) are given per tensor; a stride triple of all zeros means the
 * dense [B, H, S, d] layout. (A [B, S, H, d] caller passes
 * strides {S*H*d, d, H*d}.) Strides must be multiples of 8 elements and the
 * base pointers 16-byte aligned (else DIT_ERR_UNSUPPORTED).
 *
 * Rows s >= q_valid of Q and s >= kv_valid of K/V are tail pads: pad keys take
 * no part in any softmax (their content, even NaN or Inf, cannot change a
 * result), and pad query rows get O = +0.0 and LSE = -inf. With kv_valid == 0
 * every row gets O = 0 and LSE = -inf (-inf is the identity of the merge).
 *
 * RoPE (split halves: channel i pairs with i + d/2, i < d/2):
 *   x'_i = x_i c_i - x_{i+d/2} s_i,  x'_{i+d/2} = x_{i+d/2} c_i + x_i s_i
 * computed in fp32 from the bf16 inputs and fp32 tables, rounded once to
 * bf16 (round to nearest even). cos_q/sin_q are fp32 [s_q, d/2] tables for
 * the query rows, cos_k/sin_k fp32 [s_kv, d/2] for the key rows (for a key
 * shard, pass the table pointers offset to the shard's first row). Each pair
 * must be both NULL (no rotation) or both non-NULL. With rotation, B * H may
 * not exceed 262140 (else DIT_ERR_UNSUPPORTED).
 *
 * Scores are sm_scale * <q'_i, k'_j> (sm_scale == 0 selects 1/sqrt(d); it
 * must be finite and positive). Both contractions run on bf16 MFMA with fp32
 * accumulation; softmax probabilities are rounded to bf16 before P.V.
 *
 * Outputs: O in o_dtype (DIT_BF16 for a final result, DIT_F32 for a partial
 * result that dit_lse_merge will combine), written for rows [0, s_q).
 * lse: fp32 dense [B, H, s_q], natural log, or NULL to skip it.
 *
 * workspace: device scratch for the once-per-call rotated (and normalised)
 * copies of K and Q (dense bf16 [B, H, s, d] each, when their tables or norm
 * weights are given), under the BALANCED schedule two fp32 partial-result
 * slots per workgroup (2 * CUs * (256 KB / 128 * d + 1 KB)) and one int32
 * arrival counter per query tile, under DYNAMIC (also when AUTO picks it)
 * nine int32 counters (256 bytes), and with fixed_m
 * the key and query statistics (fp32, about B*H*(s_q + 2*d + s_kv*d/256)
 * values). Required (non-NULL, 256-byte aligned, at least
 * dit_attn_workspace_size() bytes) when that size is non-zero. The caller
 * owns it; its contents need not be initialised. Calls that share one
 * workspace must not overlap.
 *
 * ws_counters_zero: the BALANCED schedule's arrival counters and the
 * DYNAMIC schedule's queue counters must be zero when the attention kernel
 * starts, and every completed call leaves them zero. With 0 the call clears them (inside the Q/K pre-pass when one runs,
 * else with one small fill kernel). With 1 the caller guarantees they are
 * zero because the workspace comes unchanged from an earlier completed call
 * with the same arguments, and the clear is skipped.
 *
 * schedule: a dit_schedule value (0 = AUTO).
 *
 * q/k RMS normalisation (optional, fused into the rotation pre-pass; the
 * per-head q/k RMSNorm that precedes RoPE in FLUX and Wan, Difflet PR #153
 * split-RoPE commits): with q_norm_w (k_norm_w) non-NULL, each head vector
 * of Q (K) is first replaced by
 *   y_c = x_c / sqrt(mean_c' x_c'^2 + norm_eps) * w_c
 * in fp32 from the bf16 input, then rotated (when its tables are given) and
 * rounded once to bf16. w: device fp32 [d] in the channel order of Q/K (the
 * split-halves order: permute it with the channels), 16-byte aligned.
 * norm_eps must be finite and >= 0 (0 with an all-zero row gives NaN there).
 *
 * Segments (the ring layout: maxdiffusion PR #491 pads each ring segment at
 * its own tail): with kv_seg_len > 0, K/V hold s_kv / kv_seg_len segments of
 * kv_seg_len rows and kv_valid counts the real rows at the head of EACH
 * segment; key j is real iff j mod kv_seg_len < kv_valid. Likewise
 * q_seg_len > 0 makes query row i real iff i mod q_seg_len < q_valid. One
 * softmax runs over all real keys of all segments; pad query rows get O = +0
 * and LSE = -inf. s must be a multiple of its segment length and valid <=
 * segment length (else DIT_ERR_INVALID); kv_seg_len must be a multiple of 64
 * (segmented calls run PER_QTILE whatever the schedule asks).
 *
 * fixed_m selects the fixed-m softmax (maxdiffusion PR #491; the bound is
 * not printed there, the plain reading is used): 1 = on, 2 = off (online
 * softmax), 0 = AUTO: on where a head has at least 32768 real keys (then its
 * statistics passes cost a small part of the call and the loop without a
 * running maximum wins, e.g. the Wan 720p shard), off below. When on: before the attention kernel,
 * passes over K (and Q) compute, over the real keys of each head, the key
 * mean kbar and R = max_j |k_j - kbar|, and for every query row the bound
 *   m_i = sm_scale * (q_i . kbar + |q_i| R) >= every score of row i
 * (from the rotated / normalised bf16 Q and K). A q-tile whose real rows all
 * have 2 sm_scale |q_i| R <= 96 ln 2 uses m_i as its fixed softmax maximum
 * (no running max, no rescale); any other q-tile keeps the online softmax.
 * Results agree with the online softmax to rounding and are reproducible
 * run to run. Needs workspace; runs PER_QTILE whatever the schedule asks. It
 * pays for itself only on long key ranges.
 */
typedef struct dit_attn_desc {
  int32_t B, H, d;               /* d in {64, 128}, else DIT_ERR_UNSUPPORTED */
  int32_t s_q, s_kv;             /* rows present in Q/O and in K/V (padded lengths) */
  int32_t q_valid, kv_valid;     /* real tokens, 0 <= valid <= s */
  int32_t o_dtype;               /* dit_dtype */
  const void *q, *k, *v;         /* bf16 */
  void *o;                       /* bf16 or fp32 per o_dtype */
  float *lse;                    /* fp32 [B, H, s_q] or NULL */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];  /* (b, h, s) in elements */
  float sm_scale;
  const float *cos_q, *sin_q;    /* fp32 [s_q, d/2] or NULL */
  const float *cos_k, *sin_k;    /* fp32 [s_kv, d/2] or NULL */
  void *workspace;
  size_t workspace_bytes;
  int32_t schedule;              /* dit_schedule */
  const float *q_norm_w, *k_norm_w;  /* fp32 [d] RMSNorm weights or NULL (no norm) */
  float norm_eps;
  int32_t q_seg_len, kv_seg_len; /* 0, or segment length: see "Segments" above */
  int32_t fixed_m;               /* 0 = AUTO, 1 = fixed-m, 2 = online softmax: see above */
  int32_t ws_counters_zero;      /* 1: the workspace's Stream-K counters are known zero; see above */
} dit_attn_desc;

/* Bytes of workspace dit_attn_fwd needs for `desc` (0 when neither Q nor K
 * is rotated or normalised, the schedule needs no partial results and
 * the fixed-m softmax is off, or when kv_valid is 0). Under BALANCED and AUTO the schedule
 * and the size depend on the current device's compute-unit count
 * (DIT_ERR_HIP if it cannot be queried). */
DIT_API int dit_attn_workspace_size(const dit_attn_desc *desc, size_t *bytes);

/* Attention forward with fused RoPE and exact pad-key masking; see above. */
DIT_API int dit_attn_fwd(const dit_attn_desc *desc, void *stream);

/* Size of the static device scratch array behind dit_attn_fwd_noalloc. */
#define DIT_NOALLOC_SCRATCH_BYTES (128u << 20)

/*
 * dit_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels as dit_attn_fwd with the same desc, but
 * the workspace is a static device array of the library,
 * DIT_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the library's load
 * on that GPU until the process ends; desc->workspace, workspace_bytes and
 * ws_counters_zero are ignored. The caller still owns and passes Q, K, V, O,
 * LSE and the tables. Nothing is allocated or freed: the array's device
 * address is looked up once per device (hipGetSymbolAddress, with the device
 * current) and cached.
 * A call whose workspace (dit_attn_workspace_size) exceeds the array returns
 * DIT_ERR_UNSUPPORTED before any launch (e.g. the Wan 720p shard's 388 MB of
 * rotated Q and K). Every call on one GPU uses the same array, which keeps
 * the previous call's contents (the schedule counters are cleared by each
 * call): calls that may overlap on one GPU (other streams, other threads)
 * race on it and must be serialised by the caller. Status codes otherwise
 * as dit_attn_fwd; DIT_ERR_HIP if the array's address cannot be resolved.
 */
DIT_API int dit_attn_fwd_noalloc(const dit_attn_desc *desc, void *stream);

/*
 * Merge n_parts partial results over disjoint key shards of the same queries
 * (mstar PR #376, attention_over_sharded_keys). For every row (b, h, i):
 *   M = max_k L_k;  w_k = exp(L_k - M);  L = M + ln(sum_k w_k);
 *   O = sum_k w_k O_k / sum_k w_k.
 * A row whose parts are all -inf gives O = 0, L = -inf; rows i >= q_valid
 * give O = 0, L = -inf. o_parts / lse_parts are HOST arrays of n_parts device
 * pointers to dense [B, H, S, d] (part_dtype) and [B, H, S] fp32 tensors.
 * o_out is dense [B, H, S, d] in out_dtype; lse_out fp32 [B, H, S] or NULL.
 * 1 <= n_parts <= 16; d in {64, 128}.
 */
DIT_API int dit_lse_merge(int n_parts, const void *const *o_parts, const float *const *lse_parts,
                  int part_dtype, int B, int H, int S, int d, int q_valid,
                  void *o_out, int out_dtype, float *lse_out, void *stream);

/*
 * Split-halves RoPE tables from integer positions (Difflet PR #153, FLUX
 * split-RoPE commit: tables built once per forward). pos: device int32
 * [S, n_axes]. axis_channels: HOST array of n_axes even channel counts
 * summing to d (t, h, w order). Axis a owns d/2 pair columns
 * [P_a, P_a + c_a/2) with P_a = sum_{b<a} c_b/2, and pair j of axis a turns at
 * theta^(-2j/c_a) per position step:
 *   cos_out[s, P_a + j] = cos(pos[s, a] * theta^(-2j/c_a)), sin_out likewise.
 * Angles and sines are evaluated in fp64 and rounded to fp32. Position 0 is
 * the identity rotation (text tokens, pad rows). cos_out/sin_out: device fp32
 * [S, d/2]. 1 <= n_axes <= 8, 2 <= d <= 256 (else DIT_ERR_INVALID);
 * S * d/2 >= 2^31 gives DIT_ERR_UNSUPPORTED.
 */
DIT_API int dit_rope_split_tables(const int32_t *pos, int S, int n_axes, const int32_t *axis_channels,
                          int d, float theta, float *cos_out, float *sin_out, void *stream);

/*
 * Tail padding of token rows: in [B, s_valid, row_bytes] -> out
 * [B, s_pad, row_bytes], rows >= s_valid of `out` set to zero bytes
 * (Difflet PR #153 Wan padding commit, 4680 -> 4736). Both buffers are
 * dense device memory owned by the caller; they must not alias.
 * DIT_ERR_INVALID: B < 1, s_valid < 0, s_pad < s_valid, row_bytes <= 0, a
 * required NULL pointer, in == out. DIT_ERR_UNSUPPORTED: B > 65535.
 */
DIT_API int dit_pad_tokens(const void *in, void *out, int B, int s_valid, int s_pad,
                   int64_t row_bytes, void *stream);

/*
 * Tail padding of fused token rows with the split-halves RoPE applied on the
 * way (Difflet PR #153: Wan padding commit, 4680 -> 4736, and FLUX split-RoPE
 * commit, x'_i = x_i c_i - x_{i+d/2} s_i, x'_{i+d/2} = x_{i+d/2} c_i + x_i s_i;
 * the pages fuse the rotation into the neighbouring data movement).
 * in:  device bf16 [B, s_valid, T, H, d], dense, token-major (what one
 *      all-to-all of the stacked Q, K, V hands over: T = 3);
 * out: device bf16 [B, s_pad, T, H, d], dense, owned by the caller.
 * For every real row s < s_valid the head vectors of tensors t < n_rot (Q,
 * then K) are rotated with row s of cos_t / sin_t (device fp32 [>= s_valid,
 * d/2], as dit_rope_split_tables writes them) in fp32 and rounded once to
 * bf16 (to nearest even), exactly as dit_attn_fwd's own pre-pass rotates;
 * the other tensors are copied; rows >= s_valid of `out` are zero. Feeding
 * `out` to dit_attn_fwd without tables therefore gives the same bits as
 * dit_pad_tokens followed by dit_attn_fwd with the tables.
 * DIT_ERR_INVALID: B < 1, s_valid < 0, s_pad < s_valid, T < 1, H < 1,
 * n_rot outside [0, T], a required NULL pointer, in == out, a pointer not
 * 16-byte aligned. DIT_ERR_UNSUPPORTED: d not in {64, 128}, B > 65535,
 * T * H * d/16 * s_pad >= 2^31.
 */
DIT_API int dit_pad_tokens_rope(const void *in, void *out, int B, int s_valid, int s_pad, int T, int H, int d,
                                int n_rot, const float *cos_t, const float *sin_t, void *stream);

/* Inverse of dit_pad_tokens: in [B, s_pad, row_bytes] -> out [B, s_valid, row_bytes]
 * (no in-place operation; same status codes as dit_pad_tokens). */
DIT_API int dit_unpad_tokens(const void *in, void *out, int B, int s_pad, int s_valid,
                     int64_t row_bytes, void *stream);

/* Host helper: *s_pad_out = ceil(s_valid / multiple) * multiple, the tail
 * padding plan of the pages: Difflet PR #153, Wan padding + split RoPE commit
 * (4680 tokens padded to 4736, a multiple of 128; the LTX-2 scope pads to a
 * multiple of 2*tp, 2310 -> 2312) and maxdiffusion PR #491, lane padding
 * (each shard a multiple of 128 rows, 75,600 -> 75,776 at CP=4).
 * DIT_ERR_INVALID: s_pad_out NULL, multiple <= 0, s_valid < 0, or a padded
 * length beyond INT32_MAX. No HIP call is made. */
DIT_API int dit_plan_padding(int s_valid, int multiple, int *s_pad_out);

/* Thread-local description of the last non-OK status ("" if none). */
DIT_API const char *dit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H_ */
