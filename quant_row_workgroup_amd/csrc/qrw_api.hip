// qrw_api.hip -- the C ABI (include/qrw.h): argument validation with integer
// compares only, then one launch on the caller's stream.
//
// The checks are the applicable ones of the host-side launcher checks listed
// on the page "TileLang kernel DSL in DeepSeek-V4" (host code generation:
// argument count/type, null pointers, dtype, shape, stride), done in plain
// C++ before anything is enqueued; a failing call has no side effects.
// Device identity is the caller's business (the pointers and the stream
// already name a device).
#include <cmath>
#include <cstdint>

#include "qrw.h"
#include "qrw_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_16bit(int dtype) { return dtype == QRW_F16 || dtype == QRW_BF16; }

bool cs_ok(int dtype, int cs_dtype) { return cs_dtype == QRW_F32 || cs_dtype == dtype; }

// Byte range [lo, hi) touched by `rows` rows of `n` elements `stride` apart.
struct Span {
  uintptr_t lo, hi;
};
Span span_of(const void* p, int64_t rows, int64_t n, int64_t stride, int64_t elt) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)(((rows - 1) * stride + n) * elt)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// The bytes that `rows` rows of `n` elements `stride` apart span must fit the
// address space (2^56 bytes here); nothing larger describes memory, and the
// span arithmetic above could overflow.  Formed in 128 bits.
constexpr int64_t kMaxExtent = (int64_t)1 << 56;
bool extent_ok(int64_t rows, int64_t n, int64_t stride, int64_t elt) {
  if (rows <= 0) return true;
  return ((__int128)(rows - 1) * stride + n) * elt <= (__int128)kMaxExtent;
}

// y may equal x exactly (same base, same stride); any other overlap is refused.
int check_alias(const void* x, int64_t xs, const void* y, int64_t ys, int64_t rows, int64_t n,
                int64_t elt) {
  if (x == y) return xs == ys ? QRW_OK : QRW_ERR_ALIAS;
  if (overlap(span_of(x, rows, n, xs, elt), span_of(y, rows, n, ys, elt))) return QRW_ERR_ALIAS;
  return QRW_OK;
}

// An input that must not be written (weights, tables) may not overlap the output.
int check_disjoint(const void* in, int64_t in_bytes, Span out) {
  if (!in) return QRW_OK;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(in);
  return overlap({lo, lo + (uintptr_t)in_bytes}, out) ? QRW_ERR_ALIAS : QRW_OK;
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

// Shape, dtype and scalar checks of a row operator (pointers are checked
// separately, after the empty case: a zero-row tensor may have no storage).
int check_row_shape(int64_t rows, int64_t n, int64_t max_n, int64_t xs, int64_t ys, int dtype,
                    float eps) {
  if (!is_16bit(dtype)) return QRW_ERR_DTYPE;
  if (rows < 0 || n < 1 || n > max_n) return QRW_ERR_SHAPE;
  // grid.x limit: four rows per workgroup, or one row per workgroup for long rows
  if (rows > (n > 8 * qrw::kOneWaveGranules ? (int64_t)0x7FFFFFFF : (int64_t)0x7FFFFFFF * 4))
    return QRW_ERR_SHAPE;
  if (xs < n || ys < n || xs % 8 != 0 || ys % 8 != 0) return QRW_ERR_STRIDE;
  if (!extent_ok(rows, n, xs, 2) || !extent_ok(rows, n, ys, 2)) return QRW_ERR_STRIDE;
  if (!eps_ok(eps)) return QRW_ERR_VALUE;
  return QRW_OK;
}

int check_heads(int64_t tokens, int64_t heads, int64_t head_dim, int64_t rope_dim) {
  if (tokens < 0 || heads < 1 || head_dim < 8 || head_dim % 8 != 0) return QRW_ERR_SHAPE;
  if (rope_dim < 16 || rope_dim % 16 != 0 || rope_dim > head_dim) return QRW_ERR_SHAPE;
  if (heads > QRW_MAX_ROW || head_dim > QRW_MAX_ROW || heads * head_dim > QRW_MAX_ROW)
    return QRW_ERR_SHAPE;
  if (tokens > (int64_t)0x7FFFFFFF * 4) return QRW_ERR_SHAPE;
  return QRW_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? QRW_OK : QRW_ERR_LAUNCH; }

bool is_dtype(int dtype) { return dtype == QRW_F16 || dtype == QRW_BF16 || dtype == QRW_F32; }
int64_t elt_size(int dtype) { return dtype == QRW_F32 ? 4 : 2; }

constexpr int64_t kMaxFlat = (int64_t)1 << 40;

// The elementwise family: y may be x (or b) exactly when it has the same dtype
// (each element is read before the same lane writes it); any other overlap of
// an output with an input is refused.
int ew_checked(const void* x, const void* b, void* y, int64_t n, float alpha, int x_dtype,
               int y_dtype, void* stream) {
  if (!is_dtype(x_dtype) || !is_dtype(y_dtype)) return QRW_ERR_DTYPE;
  if (n < 0 || n > kMaxFlat) return QRW_ERR_SHAPE;
  if (n == 0) return QRW_OK;
  if (!x || !y) return QRW_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (b && !aligned16(b))) return QRW_ERR_ALIGN;
  const Span ys = span_of(y, 1, n, 0, elt_size(y_dtype));
  for (const void* in : {x, b}) {
    if (!in) continue;
    if (in == y && x_dtype == y_dtype) continue;
    if (overlap(span_of(in, 1, n, 0, elt_size(x_dtype)), ys)) return QRW_ERR_ALIAS;
  }
  return finish(qrw::launch_ew(x, b, y, n, alpha, x_dtype, y_dtype,
                               static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int rmsnorm_fwd(const void* x, const void* weight, void* y, int64_t rows, int64_t n,
                int64_t x_row_stride, int64_t y_row_stride, int dtype, float eps,
                void* stream) {
  int st = check_row_shape(rows, n, QRW_MAX_ROW_SPLIT, x_row_stride, y_row_stride, dtype, eps);
  if (st != QRW_OK) return st;
  if (rows == 0) return QRW_OK;
  if (!x || !y) return QRW_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (weight && !aligned16(weight))) return QRW_ERR_ALIGN;
  st = check_alias(x, x_row_stride, y, y_row_stride, rows, n, 2);
  if (st != QRW_OK) return st;
  st = check_disjoint(weight, 2 * n, span_of(y, rows, n, y_row_stride, 2));
  if (st != QRW_OK) return st;
  return finish(qrw::launch_rmsnorm(x, weight, y, rows, n, x_row_stride, y_row_stride, dtype,
                                    eps, static_cast<hipStream_t>(stream)));
}

int layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                  int64_t n, int64_t x_row_stride, int64_t y_row_stride, int dtype, float eps,
                  void* stream) {
  int st = check_row_shape(rows, n, QRW_MAX_ROW_RESIDENT, x_row_stride, y_row_stride, dtype, eps);
  if (st != QRW_OK) return st;
  if (rows == 0) return QRW_OK;
  if (!x || !y) return QRW_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (gamma && !aligned16(gamma)) ||
      (beta && !aligned16(beta)))
    return QRW_ERR_ALIGN;
  st = check_alias(x, x_row_stride, y, y_row_stride, rows, n, 2);
  if (st != QRW_OK) return st;
  const Span out = span_of(y, rows, n, y_row_stride, 2);
  if (check_disjoint(gamma, 2 * n, out) != QRW_OK || check_disjoint(beta, 2 * n, out) != QRW_OK)
    return QRW_ERR_ALIAS;
  return finish(qrw::launch_layernorm(x, gamma, beta, y, rows, n, x_row_stride, y_row_stride,
                                      dtype, eps, static_cast<hipStream_t>(stream)));
}

static int rope_common(const void* x, const void* cos, const void* sin, void* y, int64_t tokens,
                       int64_t heads, int64_t head_dim, int64_t rope_dim, int64_t xs,
                       int64_t ys, int dtype, int cs_dtype, bool neox, void* stream) {
  if (!is_16bit(dtype) || !cs_ok(dtype, cs_dtype)) return QRW_ERR_DTYPE;
  int st = check_heads(tokens, heads, head_dim, rope_dim);
  if (st != QRW_OK) return st;
  const int64_t n = heads * head_dim;
  if (xs < n || ys < n || xs % 8 != 0 || ys % 8 != 0) return QRW_ERR_STRIDE;
  if (!extent_ok(tokens, n, xs, 2) || !extent_ok(tokens, n, ys, 2)) return QRW_ERR_STRIDE;
  if (tokens == 0) return QRW_OK;
  if (!x || !y || !cos || !sin) return QRW_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(cos) || !aligned16(sin))
    return QRW_ERR_ALIGN;
  st = check_alias(x, xs, y, ys, tokens, n, 2);
  if (st != QRW_OK) return st;
  const int64_t tab = tokens * (rope_dim / 2) * (cs_dtype == QRW_F32 ? 4 : 2);
  const Span out = span_of(y, tokens, n, ys, 2);
  if (check_disjoint(cos, tab, out) != QRW_OK || check_disjoint(sin, tab, out) != QRW_OK)
    return QRW_ERR_ALIAS;
  return finish(qrw::launch_rope(x, cos, sin, y, tokens, heads, head_dim, rope_dim, xs, ys,
                                 dtype, cs_dtype, neox, static_cast<hipStream_t>(stream)));
}

int rope_apply_interleaved(const void* x, const void* cos, const void* sin, void* y,
                           int64_t tokens, int64_t heads, int64_t head_dim, int64_t rope_dim,
                           int64_t x_token_stride, int64_t y_token_stride, int dtype,
                           int cs_dtype, void* stream) {
  return rope_common(x, cos, sin, y, tokens, heads, head_dim, rope_dim, x_token_stride,
                     y_token_stride, dtype, cs_dtype, false, stream);
}

int rope_apply_neox(const void* x, const void* cos, const void* sin, void* y, int64_t tokens,
                    int64_t heads, int64_t head_dim, int64_t rope_dim, int64_t x_token_stride,
                    int64_t y_token_stride, int dtype, int cs_dtype, void* stream) {
  return rope_common(x, cos, sin, y, tokens, heads, head_dim, rope_dim, x_token_stride,
                     y_token_stride, dtype, cs_dtype, true, stream);
}

static int fused_entry(const void* x, const void* weight, const void* cos, const void* sin,
                       uint8_t* q, float* scales, int64_t tokens, int64_t heads,
                       int64_t head_dim, int64_t rope_dim, int64_t x_token_stride,
                       int64_t q_token_stride, int dtype, int cs_dtype, int neox, float eps,
                       bool round_mid, void* stream) {
  if (!is_16bit(dtype) || !cs_ok(dtype, cs_dtype)) return QRW_ERR_DTYPE;
  int st = check_heads(tokens, heads, head_dim, rope_dim);
  if (st != QRW_OK) return st;
  const int64_t n = heads * head_dim;
  if (x_token_stride < n || x_token_stride % 8 != 0) return QRW_ERR_STRIDE;
  if (q_token_stride < n || q_token_stride % 8 != 0) return QRW_ERR_STRIDE;
  if (!extent_ok(tokens, n, x_token_stride, 2) || !extent_ok(tokens, n, q_token_stride, 1))
    return QRW_ERR_STRIDE;
  if (!eps_ok(eps)) return QRW_ERR_VALUE;
  if (neox != 0 && neox != 1) return QRW_ERR_VALUE;
  if (tokens == 0) return QRW_OK;
  if (!x || !cos || !sin || !q || !scales) return QRW_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(cos) || !aligned16(sin) ||
      (weight && !aligned16(weight)) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return QRW_ERR_ALIGN;
  const Span qspan = span_of(q, tokens, n, q_token_stride, 1);
  const uintptr_t s_lo = reinterpret_cast<uintptr_t>(scales);
  const Span sspan = {s_lo, s_lo + (uintptr_t)(tokens * 4)};
  if (overlap(qspan, sspan)) return QRW_ERR_ALIAS;
  const Span xspan = span_of(x, tokens, n, x_token_stride, 2);
  const int64_t tab = tokens * (rope_dim / 2) * (cs_dtype == QRW_F32 ? 4 : 2);
  const void* ins[3] = {weight, cos, sin};
  const int64_t inb[3] = {2 * n, tab, tab};
  for (int i = 0; i < 3; ++i) {
    if (check_disjoint(ins[i], inb[i], qspan) != QRW_OK) return QRW_ERR_ALIAS;
    if (check_disjoint(ins[i], inb[i], sspan) != QRW_OK) return QRW_ERR_ALIAS;
  }
  if (overlap(xspan, qspan) || overlap(xspan, sspan)) return QRW_ERR_ALIAS;
  return finish(qrw::launch_rmsnorm_rope_fp8(x, weight, cos, sin, q, scales, tokens, heads,
                                             head_dim, rope_dim, x_token_stride,
                                             q_token_stride, dtype, cs_dtype, neox == 1, eps,
                                             round_mid, static_cast<hipStream_t>(stream)));
}

int rmsnorm_rope_fp8_fwd(const void* x, const void* weight, const void* cos, const void* sin,
                         uint8_t* q, float* scales, int64_t tokens, int64_t heads,
                         int64_t head_dim, int64_t rope_dim, int64_t x_token_stride,
                         int64_t q_token_stride, int dtype, int cs_dtype, int neox, float eps,
                         void* stream) {
  return fused_entry(x, weight, cos, sin, q, scales, tokens, heads, head_dim, rope_dim,
                     x_token_stride, q_token_stride, dtype, cs_dtype, neox, eps, false, stream);
}

int rmsnorm_rope_fp8_rounded_fwd(const void* x, const void* weight, const void* cos,
                                 const void* sin, uint8_t* q, float* scales, int64_t tokens,
                                 int64_t heads, int64_t head_dim, int64_t rope_dim,
                                 int64_t x_token_stride, int64_t q_token_stride, int dtype,
                                 int cs_dtype, int neox, float eps, void* stream) {
  return fused_entry(x, weight, cos, sin, q, scales, tokens, heads, head_dim, rope_dim,
                     x_token_stride, q_token_stride, dtype, cs_dtype, neox, eps, true, stream);
}

int act_quant_fp8_fwd(const void* x, uint8_t* q, float* scales, int64_t rows, int64_t n,
                      int64_t group, int64_t x_row_stride, int64_t q_row_stride, int dtype,
                      void* stream) {
  if (!is_16bit(dtype)) return QRW_ERR_DTYPE;
  if (rows < 0 || n < 8 || n % 8 != 0 || n > QRW_MAX_ROW_RESIDENT) return QRW_ERR_SHAPE;
  if (rows > (int64_t)0x7FFFFFFF * 4) return QRW_ERR_SHAPE;
  // rows longer than QRW_MAX_ROW: one workgroup per row (per token), or up to
  // 32 waves per row (per group)
  if (n > QRW_MAX_ROW && rows > (int64_t)0x7FFFFFFF / 8) return QRW_ERR_SHAPE;
  const bool pow2_group = group >= 8 && group <= 512 && (group & (group - 1)) == 0;
  if (group != n && !(pow2_group && n % group == 0)) return QRW_ERR_SHAPE;
  if (x_row_stride < n || x_row_stride % 8 != 0) return QRW_ERR_STRIDE;
  if (q_row_stride < n || q_row_stride % 8 != 0) return QRW_ERR_STRIDE;
  if (!extent_ok(rows, n, x_row_stride, 2) || !extent_ok(rows, n, q_row_stride, 1))
    return QRW_ERR_STRIDE;
  if (rows == 0) return QRW_OK;
  if (!x || !q || !scales) return QRW_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return QRW_ERR_ALIGN;
  const Span qspan = span_of(q, rows, n, q_row_stride, 1);
  const uintptr_t s_lo = reinterpret_cast<uintptr_t>(scales);
  const Span sspan = {s_lo, s_lo + (uintptr_t)(rows * (n / group) * 4)};
  const Span xspan = span_of(x, rows, n, x_row_stride, 2);
  if (overlap(qspan, sspan) || overlap(xspan, qspan) || overlap(xspan, sspan)) return QRW_ERR_ALIAS;
  return finish(qrw::launch_act_quant_fp8(x, q, scales, rows, n, group, x_row_stride,
                                          q_row_stride, dtype, static_cast<hipStream_t>(stream)));
}

int qk_norm_rope_fwd(void* qkv, const void* q_weight, const void* k_weight, const void* cos,
                     const void* sin, int64_t tokens, int64_t q_heads, int64_t kv_heads,
                     int64_t head_dim, int64_t rope_dim, int64_t token_stride, int dtype,
                     int cs_dtype, int neox, float eps, void* stream) {
  if (!is_16bit(dtype) || !cs_ok(dtype, cs_dtype)) return QRW_ERR_DTYPE;
  if (tokens < 0 || q_heads < 1 || kv_heads < 0) return QRW_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return QRW_ERR_SHAPE;
  if (rope_dim < 16 || rope_dim > head_dim || (rope_dim & (rope_dim - 1)) != 0)
    return QRW_ERR_SHAPE;
  if (q_heads > (1 << 16) || kv_heads > (1 << 16)) return QRW_ERR_SHAPE;
  const int64_t n = (q_heads + 2 * kv_heads) * head_dim;
  if (tokens > (int64_t)0x7FFFFFFF) return QRW_ERR_SHAPE;
  if (token_stride < n || token_stride % 8 != 0) return QRW_ERR_STRIDE;
  if (!extent_ok(tokens, n, token_stride, 2)) return QRW_ERR_STRIDE;
  if (!eps_ok(eps)) return QRW_ERR_VALUE;
  if (neox != 0 && neox != 1) return QRW_ERR_VALUE;
  if (tokens == 0) return QRW_OK;
  if (!qkv || !cos || !sin) return QRW_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(cos) || !aligned16(sin) ||
      (q_weight && !aligned16(q_weight)) || (k_weight && !aligned16(k_weight)))
    return QRW_ERR_ALIGN;
  const Span out = span_of(qkv, tokens, (q_heads + kv_heads) * head_dim, token_stride, 2);
  const int64_t tab = tokens * (rope_dim / 2) * (cs_dtype == QRW_F32 ? 4 : 2);
  if (check_disjoint(q_weight, 2 * head_dim, out) != QRW_OK ||
      check_disjoint(k_weight, 2 * head_dim, out) != QRW_OK ||
      check_disjoint(cos, tab, out) != QRW_OK || check_disjoint(sin, tab, out) != QRW_OK)
    return QRW_ERR_ALIAS;
  // chunks of one token row: (q_heads + kv_heads) * head_dim / 1024, rounded up
  if (tokens * (((q_heads + kv_heads) * head_dim + 1023) / 1024) > (int64_t)0x7FFFFFFF * 4)
    return QRW_ERR_SHAPE;
  return finish(qrw::launch_qk_norm_rope(qkv, q_weight, k_weight, cos, sin, tokens, q_heads,
                                         kv_heads, head_dim, rope_dim, token_stride, dtype,
                                         cs_dtype, neox == 1, eps,
                                         static_cast<hipStream_t>(stream)));
}

int qk_norm_rope_fp8_kv_fwd(void* qkv, const void* q_weight, const void* k_weight,
                            const void* cos, const void* sin, uint8_t* k_cache, uint8_t* v_cache,
                            float* k_scales, float* v_scales, const int64_t* slots,
                            int64_t num_slots, int64_t tokens, int64_t q_heads, int64_t kv_heads,
                            int64_t head_dim, int64_t rope_dim, int64_t token_stride,
                            int64_t cache_stride, int dtype, int cs_dtype, int neox, float eps,
                            void* stream) {
  if (!is_16bit(dtype) || !cs_ok(dtype, cs_dtype)) return QRW_ERR_DTYPE;
  if (tokens < 0 || q_heads < 1 || kv_heads < 1 || num_slots < 0) return QRW_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return QRW_ERR_SHAPE;
  if (rope_dim < 16 || rope_dim > head_dim || (rope_dim & (rope_dim - 1)) != 0)
    return QRW_ERR_SHAPE;
  if (q_heads > (1 << 16) || kv_heads > (1 << 16)) return QRW_ERR_SHAPE;
  if (tokens > (int64_t)0x7FFFFFFF) return QRW_ERR_SHAPE;
  if (!slots && num_slots < tokens) return QRW_ERR_SHAPE;  // token t goes to row t
  const int64_t n = (q_heads + 2 * kv_heads) * head_dim;
  const int64_t kvn = kv_heads * head_dim;
  if (token_stride < n || token_stride % 8 != 0) return QRW_ERR_STRIDE;
  if (cache_stride < kvn || cache_stride % 8 != 0) return QRW_ERR_STRIDE;
  // (the cache extent also bounds the scale arrays: 4 * num_slots * kv_heads
  // bytes is less than num_slots * kvn, since head_dim >= 64)
  if (!extent_ok(tokens, n, token_stride, 2) || !extent_ok(num_slots, kvn, cache_stride, 1))
    return QRW_ERR_STRIDE;
  if (!eps_ok(eps)) return QRW_ERR_VALUE;
  if (neox != 0 && neox != 1) return QRW_ERR_VALUE;
  if (tokens == 0) return QRW_OK;
  if (!qkv || !cos || !sin || !k_cache || !v_cache || !k_scales || !v_scales) return QRW_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(cos) || !aligned16(sin) || !aligned16(k_cache) ||
      !aligned16(v_cache) || (q_weight && !aligned16(q_weight)) ||
      (k_weight && !aligned16(k_weight)) || (reinterpret_cast<uintptr_t>(k_scales) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(v_scales) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(slots) & 7u) != 0)
    return QRW_ERR_ALIGN;
  // outputs (and the rows the kernel reads, which hold the q output) are pairwise
  // disjoint; read-only inputs overlap none of them
  Span out[5];
  int nout = 0;
  out[nout++] = span_of(qkv, tokens, n, token_stride, 2);
  if (num_slots > 0) {
    out[nout++] = span_of(k_cache, num_slots, kvn, cache_stride, 1);
    out[nout++] = span_of(v_cache, num_slots, kvn, cache_stride, 1);
    out[nout++] = span_of(k_scales, 1, num_slots * kv_heads, 0, 4);
    out[nout++] = span_of(v_scales, 1, num_slots * kv_heads, 0, 4);
  }
  for (int i = 0; i < nout; ++i)
    for (int k = i + 1; k < nout; ++k)
      if (overlap(out[i], out[k])) return QRW_ERR_ALIAS;
  const int64_t tab = tokens * (rope_dim / 2) * (cs_dtype == QRW_F32 ? 4 : 2);
  for (int i = 0; i < nout; ++i)
    if (check_disjoint(q_weight, 2 * head_dim, out[i]) != QRW_OK ||
        check_disjoint(k_weight, 2 * head_dim, out[i]) != QRW_OK ||
        check_disjoint(cos, tab, out[i]) != QRW_OK || check_disjoint(sin, tab, out[i]) != QRW_OK ||
        check_disjoint(slots, 8 * tokens, out[i]) != QRW_OK)
      return QRW_ERR_ALIAS;
  if (tokens * ((n + 1023) / 1024) > (int64_t)0x7FFFFFFF * 4) return QRW_ERR_SHAPE;
  return finish(qrw::launch_qk_norm_rope_fp8_kv(
      qkv, q_weight, k_weight, cos, sin, k_cache, v_cache, k_scales, v_scales, slots, num_slots,
      tokens, q_heads, kv_heads, head_dim, rope_dim, token_stride, cache_stride, dtype, cs_dtype,
      neox == 1, eps, static_cast<hipStream_t>(stream)));
}

int ew_add_fwd(const void* a, const void* b, void* y, int64_t n, int dtype, void* stream) {
  if (n > 0 && !b) return QRW_ERR_NULL;
  return ew_checked(a, b, y, n, 1.0f, dtype, dtype, stream);
}

int ew_scale_cast_fwd(const void* x, void* y, int64_t n, float alpha, int x_dtype, int y_dtype,
                      void* stream) {
  return ew_checked(x, nullptr, y, n, alpha, x_dtype, y_dtype, stream);
}

int ew_scale_add_fwd(const void* x, const void* b, void* y, int64_t n, float alpha, int dtype,
                     void* stream) {
  if (n > 0 && !b) return QRW_ERR_NULL;
  return ew_checked(x, b, y, n, alpha, dtype, dtype, stream);
}

const char* qrw_status_string(int status) {
  switch (status) {
    case QRW_OK: return "ok";
    case QRW_ERR_NULL: return "a required pointer is NULL";
    case QRW_ERR_DTYPE: return "unsupported dtype";
    case QRW_ERR_SHAPE: return "invalid or unsupported shape";
    case QRW_ERR_STRIDE: return "invalid row stride";
    case QRW_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QRW_ERR_ALIAS: return "output overlaps an input";
    case QRW_ERR_LAUNCH: return "kernel launch failed";
    case QRW_ERR_VALUE: return "scalar argument out of range";
    default: return "unknown status";
  }
}

}  // extern "C"
