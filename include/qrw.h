/*
 * qrw.h -- C ABI of the fused row-operator library (libqrw.so, gfx950).
 *
 * The operations are those defined on the page "TileLang tutorial, ch. 13:
 * elementwise, normalisation and RoPE operators" (tilelang-tutorial.huandu.me,
 * chapter 13), cited below by section:
 *   s3.2.1  reference RMSNorm and LayerNorm
 *   s3.3.1  the two RoPE pairings, the (positions, rope_dim/2) cos/sin table,
 *           and partial rotation of the tail span of a head
 *   s3.3.2  reference RoPE (fp32 math, one final cast)
 *   s3.1.5  per-token / per-group FP8 cast (amax -> scale -> clamp -> cast)
 *   s3.3.4  the fused RMSNorm + RoPE + per-token quantisation operator
 *   s3.1.1  elementwise add / scale / cast; s1.2 the scale+add scenario
 *   s2.4    cross-module fusion: per-head q/k RMSNorm + RoPE, v untouched, and
 *           the variant that writes k and v to an FP8 KV cache
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller.
 *   The library never allocates, frees or synchronises, keeps no mutable
 *   global state and is safe to call from several host threads.
 * Layout.  Row-major.  A "row" (or a token) is `n` contiguous elements; rows
 *   are `*_row_stride` ELEMENTS apart.  Heads are packed inside a token:
 *   head h occupies elements [h*head_dim, (h+1)*head_dim).
 * Granules.  Rows are moved in 16-byte granules, so row strides are
 *   multiples of 8 elements and every tensor base pointer is 16-byte aligned;
 *   row lengths are multiples of 8 except where an entry point says
 *   otherwise (rmsnorm_fwd, layernorm_fwd and the elementwise family take any
 *   length).  Weight vectors and tables are packed.  With zero rows (tokens,
 *   elements) nothing is read or written and pointers may be NULL.
 * Dtypes.  `dtype` is QRW_F16 or QRW_BF16 and applies to x, y and the weight
 *   vectors (the elementwise family also takes QRW_F32).  RoPE tables have
 *   `cs_dtype`, either QRW_F32 or equal to dtype.
 * Numerics.  Arithmetic is binary32 (binary64 for the elementwise family's
 *   16-bit outputs, except a plain 16-bit sum); every 16-bit or FP8 output is
 *   rounded once, to nearest-even.  A NaN or infinite input leaves unspecified
 *   the outputs computed from it (its row, its quantisation group or head,
 *   its rotation pair, or its element) and nothing else.
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *   asynchronous on it; argument errors are reported before anything is
 *   enqueued.
 * Errors.  Each call returns QRW_OK or a negative QRW_ERR_* code.  A call that
 *   fails validation has no side effects and launches nothing.  Empty inputs
 *   (rows or tokens == 0) are valid and launch nothing.  QRW_ERR_LAUNCH means
 *   the HIP launch itself failed (hipGetLastError after the launch).
 */
#ifndef QRW_H_
#define QRW_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum qrw_dtype { QRW_F16 = 1, QRW_BF16 = 2, QRW_F32 = 3 };

/* status codes */
enum qrw_status {
  QRW_OK = 0,
  QRW_ERR_NULL = -1,    /* a required pointer is NULL */
  QRW_ERR_DTYPE = -2,   /* unsupported dtype / cs_dtype code */
  QRW_ERR_SHAPE = -3,   /* a size is negative, not a multiple of its granule, or too large */
  QRW_ERR_STRIDE = -4,  /* a row stride is shorter than the row, not a multiple of 8, or
                           the rows it spans exceed 2^56 bytes */
  QRW_ERR_ALIGN = -5,   /* a pointer is not 16-byte aligned */
  QRW_ERR_ALIAS = -6,   /* output overlaps an input other than as an exact in-place alias */
  QRW_ERR_LAUNCH = -7,  /* the kernel launch failed */
  QRW_ERR_VALUE = -8    /* a scalar argument is out of range (eps negative or not finite) */
};

/* Largest row length, in elements, of the RoPE, fused and quantisation calls
 * (8192). */
#define QRW_MAX_ROW 8192
/* Largest row of rmsnorm_fwd / layernorm_fwd kept in registers (65536), and
 * of act_quant_fp8_fwd; a longer RMSNorm row takes two passes over x
 * (s3.2.4), up to QRW_MAX_ROW_SPLIT. */
#define QRW_MAX_ROW_RESIDENT 65536
#define QRW_MAX_ROW_SPLIT (1 << 26)

/*
 * RMSNorm forward (s3.2.1):
 *   rstd_r = 1 / sqrt( (1/n) * sum_j x[r,j]^2 + eps )
 *   y[r,j] = x[r,j] * rstd_r * weight[j]          (weight == NULL: weight = 1)
 * x, y: [rows, n] with row strides x_row_stride / y_row_stride (elements,
 * multiples of 8, so every row starts 16-byte aligned).  Any 1 <= n <=
 * QRW_MAX_ROW_SPLIT: a row whose length is not a multiple of 8 ends in a
 * partial granule that is read and written in at most three accesses of 4,
 * 2 and 1 elements (columns at and past n are never touched; the padding
 * counts as zero and the mean divides by n, s5.4).  Rows up to QRW_MAX_ROW_RESIDENT are read once; longer
 * rows are read twice (sum of squares, then the output in reverse chunk
 * order, s3.2.4).
 * weight: [n], packed, same dtype, or NULL.
 * y == x (same stride) computes in place; any other overlap is QRW_ERR_ALIAS.
 */
int rmsnorm_fwd(const void* x, const void* weight, void* y, int64_t rows, int64_t n,
                int64_t x_row_stride, int64_t y_row_stride, int dtype, float eps,
                void* stream);

/*
 * LayerNorm forward (s3.2.1, torch.nn.functional.layer_norm semantics):
 *   mu_r = (1/n) sum_j x[r,j];   var_r = (1/n) sum_j (x[r,j] - mu_r)^2  (biased)
 *   y[r,j] = (x[r,j] - mu_r) / sqrt(var_r + eps) * gamma[j] + beta[j]
 * gamma / beta: [n] or NULL (1 and 0).  Layout and aliasing as rmsnorm_fwd,
 * for 1 <= n <= QRW_MAX_ROW_RESIDENT (one read of x).
 */
int layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                  int64_t n, int64_t x_row_stride, int64_t y_row_stride, int dtype,
                  float eps, void* stream);

/*
 * RoPE, interleaved pairing (s3.3.1, s3.3.2).  x, y: [tokens, heads*head_dim]
 * with token strides (elements).  In each head the tail span of rope_dim
 * channels starting at S = head_dim - rope_dim rotates; channels before S are
 * copied unchanged.  With R = rope_dim and pair p in [0, R/2):
 *   a = S + 2p, b = S + 2p + 1,  c = cos[t, p],  s = sin[t, p]
 *   y[a] = x[a] c - x[b] s;      y[b] = x[a] s + x[b] c
 * cos, sin: [tokens, R/2] packed, cs_dtype (QRW_F32 or dtype); row t is the
 * angle table of token t, shared by all heads.
 * Requires head_dim % 8 == 0, rope_dim % 16 == 0, 16 <= rope_dim <= head_dim.
 * y == x (same stride) rotates in place; other overlap is QRW_ERR_ALIAS.
 */
int rope_apply_interleaved(const void* x, const void* cos, const void* sin, void* y,
                           int64_t tokens, int64_t heads, int64_t head_dim, int64_t rope_dim,
                           int64_t x_token_stride, int64_t y_token_stride, int dtype,
                           int cs_dtype, void* stream);

/*
 * RoPE, NeoX half-split pairing (s3.3.1, s3.3.2): as rope_apply_interleaved
 * but with a = S + p, b = S + p + R/2.
 */
int rope_apply_neox(const void* x, const void* cos, const void* sin, void* y, int64_t tokens,
                    int64_t heads, int64_t head_dim, int64_t rope_dim, int64_t x_token_stride,
                    int64_t y_token_stride, int dtype, int cs_dtype, void* stream);

/*
 * Fused RMSNorm -> RoPE -> per-token FP8 quantisation (s3.3.4 with the
 * per-token cast of s3.1.5).  Per token t, over its n = heads*head_dim channels:
 *   z      = RoPE( x[t,:] * rstd_t * weight )       (no rounding in between;
 *            RoPE on each head's tail span, pairing chosen by `neox`:
 *            1 = NeoX half-split, 0 = interleaved; formulas as above)
 *   amax_t = max_j |z_j|
 *   scales[t] = max(amax_t, 1e-4) / 448                         (binary32)
 *   q[t,j]    = E4M3FN( clamp(z_j / scales[t], -448, 448) )     (OCP FP8, RNE)
 * x: [tokens, n] with x_token_stride (elements); weight: [n] or NULL;
 * cos, sin: [tokens, rope_dim/2] (cs_dtype); q: [tokens, n] uint8 codes with
 * q_token_stride (bytes, a multiple of 8); scales: [tokens] float, 4-byte
 * aligned.  Requires n <= QRW_MAX_ROW and the head/rope constraints of RoPE.
 * Dequantisation is q * scales[t].
 */
int rmsnorm_rope_fp8_fwd(const void* x, const void* weight, const void* cos, const void* sin,
                         uint8_t* q, float* scales, int64_t tokens, int64_t heads,
                         int64_t head_dim, int64_t rope_dim, int64_t x_token_stride,
                         int64_t q_token_stride, int dtype, int cs_dtype, int neox, float eps,
                         void* stream);

/*
 * The staged form of the same operator, as s3.3.4's dataflow runs it: the
 * normalised row is written back in x's dtype and rotated there, so
 *   u = round_T( x[t,:] * rstd_t * weight )       (T = dtype, nearest-even)
 *   z = round_T( RoPE(u) )                        (unrotated channels: z = u)
 * and the scale is formed from z as in rmsnorm_rope_fp8_fwd, the codes as the
 * correctly rounded binary32 quotient z / scale.  This is the composition of
 * rmsnorm_fwd, rope_apply_* and act_quant_fp8_fwd with one group per row.
 * Both evaluate in binary32, so where an exact intermediate lies within that
 * evaluation's error of a 16-bit rounding boundary either neighbour may be
 * stored, by this call or by the three calls; elsewhere they agree.  Same
 * arguments, layout, limits and errors as rmsnorm_rope_fp8_fwd.
 */
int rmsnorm_rope_fp8_rounded_fwd(const void* x, const void* weight, const void* cos,
                                 const void* sin, uint8_t* q, float* scales, int64_t tokens,
                                 int64_t heads, int64_t head_dim, int64_t rope_dim,
                                 int64_t x_token_stride, int64_t q_token_stride, int dtype,
                                 int cs_dtype, int neox, float eps, void* stream);

/*
 * Activation quantisation to OCP E4M3FN (s3.1.5), one scale per group of
 * `group` consecutive channels of a row, or per row (group == n):
 *   amax_{r,k}   = max |x[r,j]| over group k of row r
 *   scales[r,k]  = max(amax_{r,k}, 1e-4) / 448                     (binary32)
 *   q[r,j]       = E4M3FN( clamp(x[r,j] / scales[r,k], -448, 448) )
 * x: [rows, n] with x_row_stride (elements); q: [rows, n] codes with
 * q_row_stride (bytes, a multiple of 8); scales: [rows, n / group] float,
 * packed, 4-byte aligned.  group is n, or one of 8, 16, 32, 64, 128, 256, 512
 * dividing n.  Requires n <= QRW_MAX_ROW_RESIDENT; a row longer than
 * QRW_MAX_ROW is taken by one workgroup (per token) or by waves on 4096- or
 * 2048-channel segments (per group), and then rows <= 2^31 / 8.
 * Dequantisation is q * scale.
 */
int act_quant_fp8_fwd(const void* x, uint8_t* q, float* scales, int64_t rows, int64_t n,
                      int64_t group, int64_t x_row_stride, int64_t q_row_stride, int dtype,
                      void* stream);

/*
 * Per-head QK RMSNorm + RoPE, IN PLACE on a packed QKV activation (s2.4 with
 * s3.2.1 and s3.3.1).  qkv: [tokens, (q_heads + 2*kv_heads) * head_dim] with
 * token_stride (elements); a row holds q_heads query heads, then kv_heads key
 * heads, then kv_heads value heads.  For every query (key) head of a token:
 *   rstd = 1 / sqrt( (1/head_dim) sum_j x_j^2 + eps )     over that head
 *   x   <- RoPE( x * rstd * w )   w = q_weight (k_weight) [head_dim], or NULL
 * with RoPE on the head's tail span of rope_dim channels (neox: 1 = NeoX
 * half-split, 0 = interleaved) using cos/sin [tokens, rope_dim/2] (cs_dtype).
 * Value heads are neither read nor written.  Requires head_dim in
 * {64, 128, 256} and rope_dim a power of two with 16 <= rope_dim <= head_dim.
 */
int qk_norm_rope_fwd(void* qkv, const void* q_weight, const void* k_weight, const void* cos,
                     const void* sin, int64_t tokens, int64_t q_heads, int64_t kv_heads,
                     int64_t head_dim, int64_t rope_dim, int64_t token_stride, int dtype,
                     int cs_dtype, int neox, float eps, void* stream);

/*
 * QK RMSNorm + RoPE with the quantised KV-cache write (s2.4, the cross-module
 * fusion: Q/K RMSNorm + RoPE + quantised KV-cache write).  Same row layout,
 * arithmetic and shape limits as qk_norm_rope_fwd, and kv_heads >= 1; then:
 *   q heads are written back in place into qkv (qkv's k and v columns are
 *   only read);
 *   for every k head (after its norm and rotation, unrounded) and every v
 *   head (as stored) of token t, with s = slots[t] (s = t if slots is NULL):
 *     scale = max(amax over the head, 1e-4) / 448        (float32)
 *     code_j = E4M3FN(RN_f32(value_j / scale))            (s3.1.5's cast)
 *     k_cache[s * cache_stride + h * head_dim + j] = code_j
 *     k_scales[s * kv_heads + h] = scale                  (v likewise)
 * k_cache, v_cache: num_slots rows of cache_stride bytes (>= kv_heads *
 * head_dim, multiple of 8), 16-byte aligned; k_scales, v_scales: float
 * [num_slots, kv_heads]; slots: int64 [tokens] or NULL (then num_slots >=
 * tokens).  A token whose slot is outside [0, num_slots) (e.g. -1 for
 * padding) writes nothing to the caches; its q is still written.  Two tokens
 * with the same slot race.  Outputs must not overlap one another or any
 * input (QRW_ERR_ALIAS).
 */
int qk_norm_rope_fp8_kv_fwd(void* qkv, const void* q_weight, const void* k_weight,
                            const void* cos, const void* sin, uint8_t* k_cache, uint8_t* v_cache,
                            float* k_scales, float* v_scales, const int64_t* slots,
                            int64_t num_slots, int64_t tokens, int64_t q_heads, int64_t kv_heads,
                            int64_t head_dim, int64_t rope_dim, int64_t token_stride,
                            int64_t cache_stride, int dtype, int cs_dtype, int neox, float eps,
                            void* stream);

/*
 * Elementwise family (s3.1.1: a + b and (x * alpha) cast to another dtype;
 * s1.2: the scale+add scenario y = x * a + b).  Flat arrays of n elements
 * (any n >= 0; no multiple-of-8 requirement), 16-byte aligned, F16, BF16 or
 * F32.  Each output is x * alpha + b rounded once, nearest-even, to y's
 * dtype (a float32 fma for float32 outputs; for 16-bit outputs a float64 fma
 * carried to the cast without a second rounding, or, for a plain sum of two
 * 16-bit values (alpha == 1), their float32 sum, which rounds the same way).
 * y may be exactly x (or b) when it
 * has the same dtype (in place); any other overlap of y with an input is
 * QRW_ERR_ALIAS.
 *   ew_add_fwd:        y = a + b              (a, b, y: dtype)
 *   ew_scale_cast_fwd: y = (x * alpha)        (x: x_dtype, y: y_dtype)
 *   ew_scale_add_fwd:  y = x * alpha + b      (x, b, y: dtype)
 */
int ew_add_fwd(const void* a, const void* b, void* y, int64_t n, int dtype, void* stream);
int ew_scale_cast_fwd(const void* x, void* y, int64_t n, float alpha, int x_dtype, int y_dtype,
                      void* stream);
int ew_scale_add_fwd(const void* x, const void* b, void* y, int64_t n, float alpha, int dtype,
                     void* stream);

/* Human-readable name of a status code (static storage). */
const char* qrw_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QRW_H_ */
