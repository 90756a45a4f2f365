// Host-side driver for the sanitizer build of the C-ABI library: every
// argument check of include/dit_attn.h runs with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code. Host arrays (merge part
// pointers, axis channel counts) are heap blocks of exactly the documented
// length, so a read past them is reported. Every case fails validation,
// which happens before any HIP call, so no GPU is needed. Prints "ALL OK"
// when every status and message matches.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "dit_attn.h"

static int failures = 0;

static void expect(const char *what, int got, int want, const char *needle) {
  const char *msg = dit_last_error();
  const bool ok = got == want && (needle == nullptr || std::strstr(msg, needle) != nullptr);
  if (!ok) {
    std::printf("FAIL %s: status %d (want %d), message \"%s\" (want \"%s\")\n", what, got, want, msg,
                needle ? needle : "");
    ++failures;
  }
}

static dit_attn_desc base_desc() {
  dit_attn_desc d;
  std::memset(&d, 0, sizeof d);
  d.B = 1; d.H = 2; d.d = 128; d.s_q = 256; d.s_kv = 256; d.q_valid = 256; d.kv_valid = 256;
  void *fake = reinterpret_cast<void *>(uintptr_t(0x10000000));   // never dereferenced
  d.q = d.k = d.v = fake;
  d.o = fake;
  return d;
}

int main() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();
  const float *fptr = reinterpret_cast<const float *>(uintptr_t(0x20000000));

  // --- dit_attn_fwd / dit_attn_workspace_size
  expect("null desc", dit_attn_fwd(nullptr, nullptr), DIT_ERR_INVALID, "NULL");
  struct Case { const char *name; void (*edit)(dit_attn_desc &); int want; const char *needle; };
  const Case cases[] = {
    {"d=96", [](dit_attn_desc &d) { d.d = 96; }, DIT_ERR_UNSUPPORTED, "d in {64, 128}"},
    {"d odd", [](dit_attn_desc &d) { d.d = 63; }, DIT_ERR_INVALID, "even"},
    {"q_valid > s_q", [](dit_attn_desc &d) { d.q_valid = 300; }, DIT_ERR_INVALID, "q_valid"},
    {"kv_valid < 0", [](dit_attn_desc &d) { d.kv_valid = -1; }, DIT_ERR_INVALID, "kv_valid"},
    {"B = 0", [](dit_attn_desc &d) { d.B = 0; }, DIT_ERR_INVALID, "B and H"},
    {"H huge negative", [](dit_attn_desc &d) { d.H = INT32_MIN; }, DIT_ERR_INVALID, "B and H"},
    {"q NULL", [](dit_attn_desc &d) { d.q = nullptr; }, DIT_ERR_INVALID, "q and o"},
    {"k NULL", [](dit_attn_desc &d) { d.k = nullptr; }, DIT_ERR_INVALID, "k and v"},
    {"o_dtype", [](dit_attn_desc &d) { d.o_dtype = 7; }, DIT_ERR_INVALID, "o_dtype"},
    {"scale < 0", [](dit_attn_desc &d) { d.sm_scale = -1.0f; }, DIT_ERR_INVALID, "sm_scale"},
    {"segments < 0", [](dit_attn_desc &d) { d.kv_seg_len = -1; }, DIT_ERR_INVALID, "segment lengths"},
    {"s_kv % kv_seg_len", [](dit_attn_desc &d) { d.kv_seg_len = 100; }, DIT_ERR_INVALID, "multiple of kv_seg_len"},
    {"kv_seg_len not tile", [](dit_attn_desc &d) { d.kv_seg_len = 32; d.kv_valid = 32; }, DIT_ERR_UNSUPPORTED, "key tile"},
    {"fixed_m = 3", [](dit_attn_desc &d) { d.fixed_m = 3; }, DIT_ERR_INVALID, "fixed_m"},
    {"ws_counters_zero", [](dit_attn_desc &d) { d.ws_counters_zero = 3; }, DIT_ERR_INVALID, "ws_counters_zero"},
    {"schedule", [](dit_attn_desc &d) { d.schedule = 9; }, DIT_ERR_INVALID, "schedule"},
    {"misaligned q", [](dit_attn_desc &d) { d.q = reinterpret_cast<void *>(uintptr_t(0x10000008)); }, DIT_ERR_UNSUPPORTED, "16-byte aligned"},
    {"stride not x8", [](dit_attn_desc &d) { d.q_stride[0] = 256 * 2 * 128; d.q_stride[1] = 128; d.q_stride[2] = 132; }, DIT_ERR_UNSUPPORTED, "multiples of 8"},
    {"workspace missing", [](dit_attn_desc &d) { d.cos_k = d.sin_k = reinterpret_cast<const float *>(uintptr_t(0x20000000)); }, DIT_ERR_INVALID, "workspace"},
  };
  for (const Case &c : cases) {
    dit_attn_desc d = base_desc();
    c.edit(d);
    expect(c.name, dit_attn_fwd(&d, nullptr), c.want, c.needle);
  }
  {
    dit_attn_desc d = base_desc();
    d.sm_scale = nan;
    expect("scale NaN", dit_attn_fwd(&d, nullptr), DIT_ERR_INVALID, "sm_scale");
    d = base_desc();
    d.sm_scale = inf;
    expect("scale inf", dit_attn_fwd(&d, nullptr), DIT_ERR_INVALID, "sm_scale");
    d = base_desc();
    d.cos_q = fptr;
    expect("cos_q alone", dit_attn_fwd(&d, nullptr), DIT_ERR_INVALID, "cos_q and sin_q");
    d = base_desc();
    d.q_norm_w = fptr;
    d.norm_eps = -1.0f;
    expect("norm_eps < 0", dit_attn_fwd(&d, nullptr), DIT_ERR_INVALID, "norm_eps");
    d = base_desc();
    d.k_norm_w = fptr;
    d.norm_eps = nan;
    expect("norm_eps NaN", dit_attn_fwd(&d, nullptr), DIT_ERR_INVALID, "norm_eps");
    size_t bytes = 1;
    d = base_desc();
    expect("workspace size plain", dit_attn_workspace_size(&d, &bytes), DIT_OK, nullptr);
    if (bytes != 0) { std::printf("FAIL workspace size plain: %zu\n", bytes); ++failures; }
    d.cos_k = d.sin_k = fptr;
    expect("workspace size K rotated", dit_attn_workspace_size(&d, &bytes), DIT_OK, nullptr);
    if (bytes != size_t(1) * 2 * 256 * 128 * 2) { std::printf("FAIL workspace size K: %zu\n", bytes); ++failures; }
    expect("workspace size NULL out", dit_attn_workspace_size(&d, nullptr), DIT_ERR_INVALID, nullptr);
  }

  // --- dit_lse_merge: exact-length heap arrays of part pointers
  for (int n : {1, 2, 16}) {
    const void **op = new const void *[n];
    const float **lp = new const float *[n];
    for (int k = 0; k < n; ++k) { op[k] = reinterpret_cast<void *>(uintptr_t(0x10000000)); lp[k] = fptr; }
    void *out = reinterpret_cast<void *>(uintptr_t(0x30000000));
    expect("merge d=96", dit_lse_merge(n, op, lp, DIT_F32, 1, 1, 8, 96, 8, out, DIT_BF16, nullptr, nullptr), DIT_ERR_UNSUPPORTED, "d in {64, 128}");
    expect("merge q_valid", dit_lse_merge(n, op, lp, DIT_F32, 1, 1, 8, 128, 9, out, DIT_BF16, nullptr, nullptr), DIT_ERR_INVALID, "q_valid");
    lp[n - 1] = nullptr;
    expect("merge NULL part", dit_lse_merge(n, op, lp, DIT_F32, 1, 1, 8, 128, 8, out, DIT_BF16, nullptr, nullptr), DIT_ERR_INVALID, "NULL pointer");
    lp[n - 1] = reinterpret_cast<const float *>(uintptr_t(0x20000002));
    expect("merge misaligned part", dit_lse_merge(n, op, lp, DIT_F32, 1, 1, 8, 128, 8, out, DIT_BF16, nullptr, nullptr), DIT_ERR_UNSUPPORTED, "aligned");
    delete[] op;
    delete[] lp;
  }
  {
    const void *op[1] = {nullptr};
    const float *lp[1] = {nullptr};
    expect("merge n=0", dit_lse_merge(0, op, lp, DIT_F32, 1, 1, 8, 128, 8, nullptr, DIT_BF16, nullptr, nullptr), DIT_ERR_INVALID, "n_parts");
    expect("merge n=17", dit_lse_merge(17, op, lp, DIT_F32, 1, 1, 8, 128, 8, nullptr, DIT_BF16, nullptr, nullptr), DIT_ERR_INVALID, "n_parts");
    expect("merge NULL arrays", dit_lse_merge(1, nullptr, nullptr, DIT_F32, 1, 1, 8, 128, 8, nullptr, DIT_BF16, nullptr, nullptr), DIT_ERR_INVALID, "host arrays");
    expect("merge dtype", dit_lse_merge(1, op, lp, 5, 1, 1, 8, 128, 8, nullptr, DIT_BF16, nullptr, nullptr), DIT_ERR_INVALID, "dtypes");
  }

  // --- dit_rope_split_tables: exact-length heap arrays of channel counts
  const int32_t *pos = reinterpret_cast<const int32_t *>(uintptr_t(0x10000000));
  float *cs = reinterpret_cast<float *>(uintptr_t(0x20000000));
  {
    int32_t *ch = new int32_t[3]{44, 42, 40};
    expect("tables sum", dit_rope_split_tables(pos, 10, 3, ch, 128, 10000.0f, cs, cs, nullptr), DIT_ERR_INVALID, "sum to 126");
    ch[2] = 41;
    expect("tables odd axis", dit_rope_split_tables(pos, 10, 3, ch, 128, 10000.0f, cs, cs, nullptr), DIT_ERR_INVALID, "even");
    ch[0] = INT32_MAX - 1; ch[1] = INT32_MAX - 1; ch[2] = 2;
    expect("tables huge axes", dit_rope_split_tables(pos, 10, 3, ch, 128, 10000.0f, cs, cs, nullptr), DIT_ERR_INVALID, "<= d");
    delete[] ch;
    int32_t *c8 = new int32_t[8]{16, 16, 16, 16, 16, 16, 16, 16};
    expect("tables theta NaN", dit_rope_split_tables(pos, 10, 8, c8, 128, nan, cs, cs, nullptr), DIT_ERR_INVALID, "theta");
    expect("tables d too big", dit_rope_split_tables(pos, 10, 8, c8, 258, 10000.0f, cs, cs, nullptr), DIT_ERR_INVALID, "d=258");
    expect("tables S too big", dit_rope_split_tables(pos, INT32_MAX, 8, c8, 128, 10000.0f, cs, cs, nullptr), DIT_ERR_UNSUPPORTED, "2^31");
    expect("tables NULL out", dit_rope_split_tables(pos, 10, 8, c8, 128, 10000.0f, nullptr, cs, nullptr), DIT_ERR_INVALID, "non-NULL");
    expect("tables S=0", dit_rope_split_tables(nullptr, 0, 8, c8, 128, 10000.0f, nullptr, nullptr, nullptr), DIT_OK, nullptr);
    delete[] c8;
    int32_t one[1] = {128};
    expect("tables n_axes=9", dit_rope_split_tables(pos, 10, 9, one, 128, 10000.0f, cs, cs, nullptr), DIT_ERR_INVALID, "n_axes");
  }

  // --- pad / unpad / plan
  void *a = reinterpret_cast<void *>(uintptr_t(0x1000)), *b = reinterpret_cast<void *>(uintptr_t(0x2000));
  expect("pad s_pad < s_valid", dit_pad_tokens(a, b, 1, 10, 5, 256, nullptr), DIT_ERR_INVALID, "s_valid");
  expect("pad alias", dit_pad_tokens(a, a, 1, 5, 10, 256, nullptr), DIT_ERR_INVALID, "alias");
  expect("pad row_bytes", dit_pad_tokens(a, b, 1, 10, 16, 0, nullptr), DIT_ERR_INVALID, "row_bytes");
  expect("pad B huge", dit_pad_tokens(a, b, 70000, 10, 16, 256, nullptr), DIT_ERR_UNSUPPORTED, "65535");
  {
    const float *t = reinterpret_cast<const float *>(uintptr_t(0x30000000));
    void *m = reinterpret_cast<void *>(uintptr_t(0x1008));
    expect("pad+rope s_pad < s_valid", dit_pad_tokens_rope(a, b, 1, 10, 5, 3, 2, 128, 2, t, t, nullptr), DIT_ERR_INVALID, "s_valid");
    expect("pad+rope n_rot > T", dit_pad_tokens_rope(a, b, 1, 10, 16, 3, 2, 128, 4, t, t, nullptr), DIT_ERR_INVALID, "n_rot");
    expect("pad+rope T = 0", dit_pad_tokens_rope(a, b, 1, 10, 16, 0, 2, 128, 0, t, t, nullptr), DIT_ERR_INVALID, "T >= 1");
    expect("pad+rope d", dit_pad_tokens_rope(a, b, 1, 10, 16, 3, 2, 96, 2, t, t, nullptr), DIT_ERR_UNSUPPORTED, "64 or 128");
    expect("pad+rope alias", dit_pad_tokens_rope(a, a, 1, 10, 16, 3, 2, 128, 2, t, t, nullptr), DIT_ERR_INVALID, "alias");
    expect("pad+rope NULL tables", dit_pad_tokens_rope(a, b, 1, 10, 16, 3, 2, 128, 2, nullptr, t, nullptr), DIT_ERR_INVALID, "cos_t");
    expect("pad+rope NULL in", dit_pad_tokens_rope(nullptr, b, 1, 10, 16, 3, 2, 128, 2, t, t, nullptr), DIT_ERR_INVALID, "in is NULL");
    expect("pad+rope NULL out", dit_pad_tokens_rope(a, nullptr, 1, 10, 16, 3, 2, 128, 2, t, t, nullptr), DIT_ERR_INVALID, "out is NULL");
    expect("pad+rope misaligned", dit_pad_tokens_rope(m, b, 1, 10, 16, 3, 2, 128, 2, t, t, nullptr), DIT_ERR_INVALID, "16-byte");
    expect("pad+rope B huge", dit_pad_tokens_rope(a, b, 70000, 10, 16, 3, 2, 128, 2, t, t, nullptr), DIT_ERR_UNSUPPORTED, "65535");
    expect("pad+rope too many tasks", dit_pad_tokens_rope(a, b, 1, 10, 1 << 24, 3, 24, 128, 2, t, t, nullptr), DIT_ERR_UNSUPPORTED, "2^31");
    expect("pad+rope empty", dit_pad_tokens_rope(nullptr, nullptr, 1, 0, 0, 3, 2, 128, 2, nullptr, nullptr, nullptr), DIT_OK, nullptr);
  }
  expect("unpad alias", dit_unpad_tokens(a, a, 1, 10, 5, 256, nullptr), DIT_ERR_INVALID, "alias");
  expect("unpad NULL", dit_unpad_tokens(nullptr, b, 1, 10, 5, 256, nullptr), DIT_ERR_INVALID, "non-NULL");
  int s_pad = 0;
  expect("plan", dit_plan_padding(4680, 128, &s_pad), DIT_OK, nullptr);
  if (s_pad != 4736) { std::printf("FAIL plan: %d\n", s_pad); ++failures; }
  expect("plan overflow", dit_plan_padding(INT32_MAX, 128, &s_pad), DIT_ERR_INVALID, nullptr);
  expect("plan multiple 0", dit_plan_padding(10, 0, &s_pad), DIT_ERR_INVALID, "multiple");
  expect("plan NULL", dit_plan_padding(10, 8, nullptr), DIT_ERR_INVALID, nullptr);

  if (failures == 0) std::printf("ALL OK\n");
  return failures == 0 ? 0 : 1;
}
