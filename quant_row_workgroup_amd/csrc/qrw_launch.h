// qrw_launch.h -- internal launchers behind the C ABI.  Arguments arrive here
// already validated (qrw_api.hip); each launcher picks a kernel instance for
// the row length and enqueues it on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qrw {

// Threads per workgroup for the row kernels: four waves, one row per wave.
constexpr int kBlock = 256;
constexpr int kRowsPerBlock = kBlock / 64;

// Row lengths of the norm kernels, in 16-byte granules: one wave holds up to
// 1024 granules (8192 elements) in registers, a workgroup of 16 waves up to
// 8192 (65536 elements); longer RMSNorm rows take the two-pass kernel.
constexpr int kOneWaveGranules = 1024;
constexpr int kResidentGranules = 8192;

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int64_t n,
                          int64_t xs, int64_t ys, int dtype, float eps, hipStream_t stream);

hipError_t launch_layernorm(const void* x, const void* g, const void* b, void* y, int64_t rows,
                            int64_t n, int64_t xs, int64_t ys, int dtype, float eps,
                            hipStream_t stream);

hipError_t launch_rope(const void* x, const void* cos, const void* sin, void* y, int64_t tokens,
                       int64_t heads, int64_t head_dim, int64_t rope_dim, int64_t xs,
                       int64_t ys, int dtype, int cs_dtype, bool neox, hipStream_t stream);

hipError_t launch_rmsnorm_rope_fp8(const void* x, const void* w, const void* cos,
                                   const void* sin, uint8_t* q, float* scales, int64_t tokens,
                                   int64_t heads, int64_t head_dim, int64_t rope_dim,
                                   int64_t xs, int64_t qs, int dtype, int cs_dtype, bool neox,
                                   float eps, bool round_mid, hipStream_t stream);

// The fused operator in the contiguous layout when every head rotates whole
// (qrw_fused_contig_{f16,bf16}.hip): rope_dim == head_dim, head_dim / 16 in
// {1, 2, 4, 8, 16}, rows of g = 1, 2, 4 or 8 blocks of 512 channels.  One
// source per x dtype, so that the library's sources compile in parallel.
hipError_t launch_rmsnorm_rope_fp8_contig_f16(const uint16_t* x, const uint16_t* w,
                                              const void* cos, const void* sin, uint8_t* q,
                                              float* scales, int64_t tokens, int64_t head_dim,
                                              int g, int64_t xs, int64_t qs, int cs_dtype,
                                              bool neox, float eps, bool round_mid,
                                              hipStream_t stream);
hipError_t launch_rmsnorm_rope_fp8_contig_bf16(const uint16_t* x, const uint16_t* w,
                                               const void* cos, const void* sin, uint8_t* q,
                                               float* scales, int64_t tokens, int64_t head_dim,
                                               int g, int64_t xs, int64_t qs, int cs_dtype,
                                               bool neox, float eps, bool round_mid,
                                               hipStream_t stream);

// The fused operator when heads rotate only their tail span, in the
// contiguous layout (qrw_fused_tail.hip): applies when rope_dim < head_dim,
// both powers of two, 16 <= rope_dim <= 256, and the row is 1, 2, 4 or 8
// blocks of 512 channels.
bool fused_tail_ok(int64_t heads, int64_t head_dim, int64_t rope_dim);
// RoPE in the contiguous lane mapping (qrw_rope_contig.hip): head_dim and
// rope_dim powers of two, 16 <= rope_dim <= min(head_dim, 256), and the row
// is 1, 2, 4, 8 or 16 blocks of 512 channels (or 3, 5, 6, 7, 10, 12, 14 for
// heads of 64 or 128; NeoX rotating whole heads).
bool rope_contig_ok(int64_t heads, int64_t head_dim, int64_t rope_dim, bool neox);
hipError_t launch_rope_contig(const void* x, const void* cos, const void* sin, void* y,
                              int64_t tokens, int64_t heads, int64_t head_dim, int64_t rope_dim,
                              int64_t xs, int64_t ys, int dtype, int cs_dtype, bool neox,
                              hipStream_t stream);
hipError_t launch_rmsnorm_rope_fp8_tail(const void* x, const void* w, const void* cos,
                                        const void* sin, uint8_t* q, float* scales,
                                        int64_t tokens, int64_t heads, int64_t head_dim,
                                        int64_t rope_dim, int64_t xs, int64_t qs, int dtype,
                                        int cs_dtype, bool neox, float eps, bool round_mid,
                                        hipStream_t stream);

hipError_t launch_act_quant_fp8(const void* x, uint8_t* q, float* scales, int64_t rows,
                                int64_t n, int64_t group, int64_t xs, int64_t qs, int dtype,
                                hipStream_t stream);

hipError_t launch_qk_norm_rope(void* qkv, const void* q_weight, const void* k_weight,
                               const void* cos, const void* sin, int64_t tokens, int64_t q_heads,
                               int64_t kv_heads, int64_t head_dim, int64_t rope_dim,
                               int64_t stride, int dtype, int cs_dtype, bool neox, float eps,
                               hipStream_t stream);

hipError_t launch_qk_norm_rope_fp8_kv(void* qkv, const void* q_weight, const void* k_weight,
                                      const void* cos, const void* sin, uint8_t* k_cache,
                                      uint8_t* v_cache, float* k_scales, float* v_scales,
                                      const int64_t* slots, int64_t num_slots, int64_t tokens,
                                      int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                                      int64_t rope_dim, int64_t stride, int64_t cache_stride,
                                      int dtype, int cs_dtype, bool neox, float eps,
                                      hipStream_t stream);

hipError_t launch_ew(const void* x, const void* b, void* y, int64_t n, float alpha, int x_dtype,
                     int y_dtype, hipStream_t stream);

// Number of "items" (pairs of granules) one token of the fused operator holds.
int64_t fused_items(int64_t heads, int64_t head_dim, int64_t rope_dim);

}  // namespace qrw
