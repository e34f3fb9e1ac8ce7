// qrw_fused_tail_bf16.hip -- the fused operator's tail-rotation kernels for
// bf16 x ("TileLang tutorial, ch. 13", s3.3.4 with s3.3.1's tail span; kernel
// and mapping in qrw_fused_tail.h).  One source per dtype so that the library
// compiles in parallel.
#include "qrw_fused_tail.h"

namespace qrw {

hipError_t launch_rmsnorm_rope_fp8_tail_bf16(const void* x, const void* w, const void* cos,
                                             const void* sin, uint8_t* q, float* scales,
                                             int64_t tokens, int64_t heads, int64_t head_dim,
                                             int64_t rope_dim, int64_t xs, int64_t qs,
                                             int cs_dtype, bool neox, float eps, bool round_mid,
                                             hipStream_t stream) {
  return tail_launch_dtype<BF16>(x, w, cos, sin, q, scales, tokens, heads, head_dim, rope_dim, xs,
                                 qs, cs_dtype, neox, eps, round_mid, stream);
}

}  // namespace qrw
