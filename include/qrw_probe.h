/*
 * qrw_probe.h -- measurement and self-check kernels that sit beside the
 * row-operator library (libqrw_probe.so).  They are not operators: the
 * benchmark uses them to bound what the hardware gives at the fused
 * operator's shape, and the GPU tests use them to check, over every input,
 * binary32 identities the quantising kernels rely on.
 *
 * Conventions as in qrw.h: plain device pointers, sizes in elements, calls
 * asynchronous on `stream` (NULL = the null stream); the library allocates,
 * frees and synchronises nothing.  Each entry point checks its arguments
 * with integer compares first and returns a negative QRW_ERR_* status (from
 * qrw.h) with nothing enqueued when one fails; otherwise it returns QRW_OK,
 * or QRW_ERR_LAUNCH if the launch failed.
 */
#ifndef QRW_PROBE_H
#define QRW_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Same-traffic copy of the fused RMSNorm -> RoPE -> per-token FP8 operator
 * ("TileLang tutorial, ch. 13", s3.3.4; byte ledger of s1.2): the same grid
 * (one wave64 per token, four tokens per 256-thread workgroup), the same
 * loads (the token's row of x as 16-byte non-temporal granules, lane l taking
 * granules l, l+64, ...; the weight granules; one 16-byte granule of the
 * token's cos and of its sin row per lane, as for heads of 128 channels) and
 * the same stores (8 bytes per lane and granule, one binary32 per token), with
 * no arithmetic beyond byte selection:
 *   q[t, j] = high byte of (x[t, j] ^ w[j] ^ cos/sin bits of lane j/8),
 *   scales[t] = bits of x[t, 0..1] XOR-reduced over the wave when
 *   `wave_dependency` is nonzero (so that, as in the operator, no store of a
 *   token is issued before the whole row has arrived), else of lane 0's first
 *   granule.
 * x: [tokens, n] 16-bit, row stride n; w: [n] 16-bit; cos, sin: [tokens, 64]
 * 16-bit; q: [tokens, n] bytes; scales: [tokens] 4-byte words.
 * n must be 4096 (the benchmark row); tokens >= 0; pointers 16-byte aligned.
 */
int qrw_probe_copy_fused_traffic(const void* x, const void* w, const void* cos,
                                 const void* sin, uint8_t* q, float* scales, int64_t tokens,
                                 int64_t n, int wave_dependency, void* stream);

/*
 * Same-traffic copy of the per-head QK RMSNorm + RoPE operators
 * ("TileLang tutorial, ch. 13", s2.4: the in-place form, and with kv != 0 the
 * form with the quantised KV-cache write) at their benchmark layout only: 32
 * query heads, 8 key and 8 value heads of 128 channels per packed row (row
 * stride 6144 16-bit channels), NeoX over the whole head.  The operators' grid
 * (one wave64 per token, four tokens per 256-thread workgroup), loads (the
 * row's q and k granules, with kv also its v granules, 16 bytes per lane and
 * instruction; per lane one granule of each weight and of the token's cos and
 * sin rows) and stores, with byte selection in place of arithmetic:
 *   every q granule (and without kv every k granule) is written back in place
 *   as x ^ weight granule ^ cos granule ^ sin granule;
 *   with kv, for a slot s = slots[t] in [0, num_slots): the k (v) granule's
 *   high bytes of x ^ weight ^ cos ^ sin (x ^ cos ^ sin) go to
 *   k_cache (v_cache) [s, 8 * granule .. +7], and each head's scale slot
 *   [s, head] receives the bits of its first lane's first word, masked with
 *   0x3FFFFFFF; other slots are skipped as in the operator.
 * qkv: [tokens, 6144] 16-bit (overwritten); q_weight, k_weight: [128] 16-bit;
 * cos, sin: [tokens, 64] 16-bit; k_cache, v_cache: [num_slots, 1024] bytes;
 * k_scales, v_scales: [num_slots, 8] 4-byte words; slots: [tokens].  Without
 * kv the cache arguments are ignored and may be NULL.  tokens >= 0; qkv,
 * weights and tables 16-byte aligned, caches 8-byte aligned.
 */
int qrw_probe_copy_qk_traffic(void* qkv, const void* q_weight, const void* k_weight,
                              const void* cos, const void* sin, uint8_t* k_cache,
                              uint8_t* v_cache, float* k_scales, float* v_scales,
                              const int64_t* slots, int64_t num_slots, int64_t tokens, int kv,
                              void* stream);

/*
 * Near-empty control: `blocks` workgroups of 256 threads; lane 0 of each wave
 * writes one 4-byte word, out[4 * block + wave] = block.  out: [4 * blocks].
 * With blocks = tokens / 4 it has the fused operator's grid.
 */
int qrw_probe_empty(uint32_t* out, int64_t blocks, void* stream);

/*
 * The fused operator's contiguous kernel (the benchmark shape's kernel: bf16
 * x, weight and cos/sin tables, NeoX, heads of 128, rows of 4096) compiled
 * with per-wave timestamps.  Arguments and results are those of
 * rmsnorm_rope_fp8_fwd with heads = 32, head_dim = rope_dim = 128, packed
 * rows; `stamps` receives 4 x uint64 per token: the constant 100 MHz clock
 * (s_memrealtime) at the wave's entry, once the row's sum of squares is known
 * (the row has arrived), after its last store is issued, and once its stores
 * have completed.  stamps: [tokens, 4].
 */
int qrw_probe_fused_timeline(const void* x, const void* w, const void* cos, const void* sin,
                             uint8_t* q, float* scales, int64_t tokens, float eps,
                             uint64_t* stamps, void* stream);

/*
 * Exhaustive sweeps of binary32 identities the quantising kernels use, over
 * the bit patterns [lo_bits, hi_bits) of positive finite binary32 values:
 *   kind 0: the reciprocal RN(1/s) formed as the hardware reciprocal refined
 *           by one Newton step, against the correctly rounded 1/s;
 *   kind 1: the scale RN(a/448) formed by Markstein's correction with the
 *           constant RN(1/448), against the correctly rounded a/448;
 *   kind 2: the device's correctly rounded binary32 division 1.0f/s, against
 *           the same reference (a check of the reference itself).
 * The reference is (float)(1.0/(double)s), resp. (float)((double)a/448.0):
 * a binary64 quotient of binary32 operands rounds innocuously to binary32.
 * Each workgroup of 256 threads covers a contiguous block of
 * 256 * per_thread patterns and writes the number of mismatches it found to
 * counts[block]; blocks = ceil((hi_bits - lo_bits) / (256 * per_thread)),
 * counts: [blocks].  No atomics, no waits across workgroups.
 * Requires lo_bits < hi_bits <= 0x7F800000, 1 <= per_thread <= 4096.
 */
int qrw_probe_sweep(int kind, uint32_t lo_bits, uint32_t hi_bits, uint32_t per_thread,
                    uint32_t* counts, int64_t blocks, void* stream);

/*
 * The same three functions on given inputs: out_recip[i] = reciprocal of
 * s[i] as the kernels form it, out_scale[i] = scale of s[i] (as an amax), for
 * i < n, so that a host can compare them with its own IEEE arithmetic.
 */
int qrw_probe_recip_values(const float* s, float* out_recip, float* out_scale, int64_t n,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QRW_PROBE_H */
