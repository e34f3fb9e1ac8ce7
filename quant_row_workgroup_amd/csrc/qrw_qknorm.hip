// qrw_qknorm.hip -- launchers of the per-head QK RMSNorm + RoPE kernels (and
// the variant with the FP8 KV-cache write); the kernel is in qrw_qknorm.h.
#include "qrw_qknorm.h"

namespace qrw {
namespace {

// Granules per lane per wave for a row of ng granules: one chunk for the
// whole row when it has at most 12 * 64 granules (the smallest width that
// holds it), else the widest width that splits the row into equal chunks,
// else 8 (the last chunk of a row is then partly idle).  Measured on MI355X:
// one wave per token, or equal chunks, are fastest; idle lane slots and
// widths above 12 (register pressure) cost time.
int pick_chunk(int ng) {
  static const int kWidths[] = {1, 2, 3, 4, 5, 6, 8, 10, 12};
  const int need = (ng + kWave - 1) / kWave;
  if (need <= 12) {
    for (int c : kWidths)
      if (c >= need) return c;
  }
  for (int i = 8; i >= 0; --i)
    if (ng % (kWave * kWidths[i]) == 0) return kWidths[i];
  return 8;
}

hipError_t qk_launch(void* qkv, const void* q_weight, const void* k_weight, const void* cos,
                     const void* sin, int64_t tokens, int64_t q_heads, int64_t kv_heads,
                     int64_t head_dim, int64_t rope_dim, int64_t stride, int dtype, int cs_dtype,
                     bool neox, float eps, KvDest kv, hipStream_t stream) {
  QkArgs a;
  a.hg = (int)(head_dim / 8);
  a.xr = (int)(rope_dim / 16);
  const int64_t heads = kv.kc ? q_heads + 2 * kv_heads : q_heads + kv_heads;
  a.ng = (int)(heads * a.hg);
  a.qg = (int)(q_heads * a.hg);
  const int gc = pick_chunk(a.ng);
  const int per_wave = kWave * gc;
  a.chunks = (a.ng + per_wave - 1) / per_wave;
  a.s0 = (int)((head_dim - rope_dim) / 8);
  a.half = (int)(rope_dim / 2);
  const int64_t waves = tokens * a.chunks;
  a.grid = dim3((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
  a.st = stream;
  a.x = static_cast<uint16_t*>(qkv);
  a.wq = static_cast<const uint16_t*>(q_weight);
  a.wk = static_cast<const uint16_t*>(k_weight);
  a.c = cos;
  a.s = sin;
  a.tokens = tokens;
  a.stride = stride;
  a.inv_n = 1.0f / (float)head_dim;  // exact: head_dim is 64, 128 or 256
  a.eps = eps;
  kv.k_end = (int)((q_heads + kv_heads) * a.hg);
  kv.kv_heads = (int)kv_heads;
  a.kv = kv;
  a.dtype = dtype;
  a.cs_dtype = cs_dtype;
  a.neox = neox;
  switch (gc) {
    case 1: qk_run_gc1(a); break;
    case 2: qk_run_gc2(a); break;
    case 3: qk_run_gc3(a); break;
    case 4: qk_run_gc4(a); break;
    case 5: qk_run_gc5(a); break;
    case 6: qk_run_gc6(a); break;
    case 8: qk_run_gc8(a); break;
    case 10: qk_run_gc10(a); break;
    default: qk_run_gc12(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_rope(void* qkv, const void* q_weight, const void* k_weight,
                               const void* cos, const void* sin, int64_t tokens, int64_t q_heads,
                               int64_t kv_heads, int64_t head_dim, int64_t rope_dim,
                               int64_t stride, int dtype, int cs_dtype, bool neox, float eps,
                               hipStream_t stream) {
  KvDest none{};
  return qk_launch(qkv, q_weight, k_weight, cos, sin, tokens, q_heads, kv_heads, head_dim,
                   rope_dim, stride, dtype, cs_dtype, neox, eps, none, stream);
}

hipError_t launch_qk_norm_rope_fp8_kv(void* qkv, const void* q_weight, const void* k_weight,
                                      const void* cos, const void* sin, uint8_t* k_cache,
                                      uint8_t* v_cache, float* k_scales, float* v_scales,
                                      const int64_t* slots, int64_t num_slots, int64_t tokens,
                                      int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                                      int64_t rope_dim, int64_t stride, int64_t cache_stride,
                                      int dtype, int cs_dtype, bool neox, float eps,
                                      hipStream_t stream) {
  KvDest kv{};
  kv.kc = k_cache;
  kv.vc = v_cache;
  kv.ks = k_scales;
  kv.vs = v_scales;
  kv.slots = slots;
  kv.num_slots = num_slots;
  kv.cache_stride = cache_stride;
  return qk_launch(qkv, q_weight, k_weight, cos, sin, tokens, q_heads, kv_heads, head_dim,
                   rope_dim, stride, dtype, cs_dtype, neox, eps, kv, stream);
}

}  // namespace qrw
