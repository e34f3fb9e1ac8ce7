// qrw_fused_tail.hip -- which fused shapes take the tail-rotation kernel, and
// its dispatch by x dtype (kernel in qrw_fused_tail.h, instantiated in
// qrw_fused_tail_{bf16,f16}.hip).
#include "qrw_fused_tail.h"

namespace qrw {

namespace {
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
}  // namespace

// Tail rotation (16 <= rope_dim < head_dim, both powers of two, rope_dim <=
// 256) on rows of 1, 2, 4 or 8 blocks of 512 channels, or of 3, 5, 6, 7 (one
// wave per token) or 10, 12, 14, 16 blocks (two) with heads of 64 or 128.
bool fused_tail_ok(int64_t heads, int64_t head_dim, int64_t rope_dim) {
  const int64_t n = heads * head_dim;
  const int64_t g = n / 512;
  if (!(rope_dim < head_dim && pow2(head_dim) && pow2(rope_dim) && rope_dim >= 16 &&
        rope_dim <= 256 && n % 512 == 0))
    return false;
  if (g == 1 || g == 2 || g == 4 || g == 8) return true;
  return (head_dim == 64 || head_dim == 128) &&
         (g == 3 || g == 5 || g == 6 || g == 7 || g == 10 || g == 12 || g == 14 || g == 16);
}

hipError_t launch_rmsnorm_rope_fp8_tail(const void* x, const void* w, const void* cos,
                                        const void* sin, uint8_t* q, float* scales,
                                        int64_t tokens, int64_t heads, int64_t head_dim,
                                        int64_t rope_dim, int64_t xs, int64_t qs, int dtype,
                                        int cs_dtype, bool neox, float eps, bool round_mid,
                                        hipStream_t stream) {
  if (dtype == 1)
    return launch_rmsnorm_rope_fp8_tail_f16(x, w, cos, sin, q, scales, tokens, heads, head_dim,
                                            rope_dim, xs, qs, cs_dtype, neox, eps, round_mid,
                                            stream);
  return launch_rmsnorm_rope_fp8_tail_bf16(x, w, cos, sin, q, scales, tokens, heads, head_dim,
                                           rope_dim, xs, qs, cs_dtype, neox, eps, round_mid,
                                           stream);
}

}  // namespace qrw
