// qrw_fused_contig_bf16.hip -- the fused RMSNorm -> RoPE -> per-token E4M3
// operator's contiguous-layout kernels for bf16 x ("TileLang tutorial,
// ch. 13", s3.3.4; kernel and layout in qrw_fused_contig.h).  One source per
// dtype so that the library compiles in parallel.
#include "qrw_fused_contig.h"
#include "qrw_launch.h"

namespace qrw {

hipError_t launch_rmsnorm_rope_fp8_contig_bf16(const uint16_t* x, const uint16_t* w,
                                                 const void* cos, const void* sin, uint8_t* q,
                                                 float* scales, int64_t tokens, int64_t head_dim,
                                                 int g, int64_t xs, int64_t qs, int cs_dtype,
                                                 bool neox, float eps, bool round_mid,
                                                 hipStream_t stream) {
  return contig_launch_dtype<BF16>(x, w, cos, sin, q, scales, tokens, head_dim, g, xs, qs, cs_dtype,
                                  neox, eps, round_mid, stream);
}

}  // namespace qrw
