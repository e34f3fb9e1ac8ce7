// qrw_probe.hip -- libqrw_probe.so: measurement and self-check kernels beside
// the row-operator library (include/qrw_probe.h).
//
// * copy_fused_traffic_kernel: the fused operator's memory traffic and grid
//   with byte selection in place of arithmetic -- the bound an operator with
//   this access structure can reach at this size.
// * copy_qk_traffic_kernel: the same for the per-head QK RMSNorm + RoPE
//   operators (in place, and with the FP8 KV-cache write) at their
//   benchmark layout.
// * empty_kernel: the same grid doing (almost) nothing -- the fixed cost of a
//   launch of that grid.
// * the fused operator's contiguous kernel with per-wave timestamps
//   (qrw_fused_contig.h, TL = true): where a launch's time goes.
// * sweep_kernel: every binary32 input of the quantisers' division-free
//   reciprocal and scale, against correctly rounded references.
#include <hip/hip_runtime.h>

#include "../qrw_device.h"
#include "../qrw_fused_contig.h"
#include "qrw.h"
#include "qrw_probe.h"

namespace qrw {
namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeRows = kProbeBlock / kWave;

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? QRW_OK : QRW_ERR_LAUNCH; }

// High bytes of the eight 16-bit elements of a granule, element k in byte k.
__device__ __forceinline__ u32x2 high_bytes(u32x4 g) {
  // v_perm_b32 selector bytes 3,1 of the second source and 3,1 of the first
  const uint32_t lo = __builtin_amdgcn_perm(g[1], g[0], 0x07050301u);
  const uint32_t hi = __builtin_amdgcn_perm(g[3], g[2], 0x07050301u);
  return (u32x2){lo, hi};
}

template <bool DEP>
__global__ __launch_bounds__(kProbeBlock) void copy_fused_traffic_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const uint16_t* cosv,
    const uint16_t* sinv, uint8_t* q, float* scales, int64_t tokens) {
  constexpr int G = 8;  // 4096 channels = 8 wave blocks of 512
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kProbeRows + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const uint16_t* xr = x + t * (int64_t)(G * 512);
  uint8_t* qr = q + t * (int64_t)(G * 512);
  u32x4 r[G], wr[G];
#pragma unroll
  for (int g = 0; g < G; ++g) r[g] = ld16_stream(xr + 8 * (kWave * g + lane));
#pragma unroll
  for (int g = 0; g < G; ++g) wr[g] = ld16(w + 8 * (kWave * g + lane));
  // one granule of the token's cos and sin rows per lane (heads of 128: lane
  // l uses granule l mod 8 of the 64-entry row)
  const u32x4 c = ld16(cosv + t * 64 + 8 * (lane & 7));
  const u32x4 s = ld16(sinv + t * 64 + 8 * (lane & 7));
  const u32x4 cs = c ^ s;
  uint32_t red = r[0][0];
  if (DEP) {
#pragma unroll
    for (int g = 1; g < G; ++g) red ^= r[g][0];
    // XOR over the wave: every store below waits for every lane's row data
    red ^= __builtin_amdgcn_update_dpp(0, red, kDppXor1, 0xF, 0xF, true);
    red ^= __builtin_amdgcn_update_dpp(0, red, kDppXor2, 0xF, 0xF, true);
    red ^= __builtin_amdgcn_update_dpp(0, red, kDppHalfMirror, 0xF, 0xF, true);
    red ^= __builtin_amdgcn_update_dpp(0, red, kDppMirror, 0xF, 0xF, true);
    red = (__builtin_amdgcn_readlane(red, 0) ^ __builtin_amdgcn_readlane(red, 16)) ^
          (__builtin_amdgcn_readlane(red, 32) ^ __builtin_amdgcn_readlane(red, 48));
  }
  if (lane == 0) scales[t] = __builtin_bit_cast(float, red & 0x3FFFFFFFu);
  const u32x4 mix = DEP ? (cs ^ (u32x4){red, red, red, red}) : cs;
#pragma unroll
  for (int g = 0; g < G; ++g) st8(qr + 8 * (kWave * g + lane), high_bytes(r[g] ^ wr[g] ^ mix));
}

// The QK operators' benchmark layout: 32 query heads, 8 key and 8 value heads
// of 128 channels (16 granules) per packed row of 6144 16-bit channels; one
// wave per token reads the q and k heads (and, with the KV write, the v heads)
// as 12 (10) granules per lane.
constexpr int kQkRowGran = 768;  // granules per packed row
constexpr int kQkQGran = 512;    // q heads
constexpr int kQkKGran = 128;    // k heads, and as many v heads
constexpr int kQkHeadGran = 16;

template <bool KV>
__global__ __launch_bounds__(kProbeBlock) void copy_qk_traffic_kernel(
    uint16_t* qkv, const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const uint16_t* cosv, const uint16_t* sinv, uint8_t* kc, uint8_t* vc, float* ks, float* vs,
    const int64_t* slots, int64_t num_slots, int64_t tokens) {
  constexpr int G = (KV ? kQkQGran + 2 * kQkKGran : kQkQGran + kQkKGran) / kWave;
  constexpr int GQ = kQkQGran / kWave;     // slots g < GQ hold q granules
  constexpr int GK = kQkKGran / kWave;     // then GK slots of k, then GK of v
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kProbeRows + (threadIdx.x >> 6);
  if (t >= tokens) return;
  uint16_t* row = qkv + t * (int64_t)(8 * kQkRowGran);
  u32x4 r[G];
#pragma unroll
  for (int g = 0; g < G; ++g) r[g] = ld16_stream(row + 8 * (kWave * g + lane));
  // a lane's place in its head fixes its weight granules and its table
  // granule (NeoX over the whole head: granule j mod 8 of the 64-entry row)
  const int j = lane & (kQkHeadGran - 1);
  const u32x4 cs = ld16(cosv + t * 64 + 8 * (j & 7)) ^ ld16(sinv + t * 64 + 8 * (j & 7));
  const u32x4 mq = ld16(wq + 8 * j) ^ cs;
  const u32x4 mk = ld16(wk + 8 * j) ^ cs;
  int64_t slot = t;
  if constexpr (KV) slot = slots[t];
  const bool cached = slot >= 0 && slot < num_slots;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int gi = kWave * g + lane;
    if (!KV || g < GQ) {
      st16_stream(row + 8 * gi, r[g] ^ (g < GQ ? mq : mk));
    } else if (cached) {
      const bool is_v = g >= GQ + GK;
      const int hg = gi - (is_v ? kQkQGran + kQkKGran : kQkQGran);  // granule inside the part
      st8_stream((is_v ? vc : kc) + slot * (8 * kQkKGran) + 8 * hg,
                 high_bytes(r[g] ^ (is_v ? cs : mk)));
      if (j == 0)
        (is_v ? vs : ks)[slot * (kQkKGran / kQkHeadGran) + hg / kQkHeadGran] =
            __builtin_bit_cast(float, r[g][0] & 0x3FFFFFFFu);
    }
  }
}

__global__ __launch_bounds__(kProbeBlock) void empty_kernel(uint32_t* out) {
  if ((threadIdx.x & (kWave - 1)) == 0)
    out[(int64_t)blockIdx.x * kProbeRows + (threadIdx.x >> 6)] = blockIdx.x;
}

template <bool NEOX>
__global__ __launch_bounds__(kWave * kContigRows) void fused_timeline_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const void* cosv, const void* sinv,
    uint8_t* q, float* scales, int64_t tokens, float eps, uint64_t* stamps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kContigRows + (threadIdx.x >> 6);
  if (t >= tokens) return;
  contig_token<BF16, BF16, NEOX, 8, true, 8, false, true>(x, w, cosv, sinv, q, scales, t, 4096,
                                                          4096, eps, lane, stamps);
}

// True when `got` is the binary32 value nearest to the binary64 value q.  (q
// is the binary64 quotient of binary32 operands; the exact quotient is never
// within 2^-49 (relative) of a binary32 rounding boundary, while q is within
// 2^-53 of it, so the nearest binary32 to q is the correctly rounded quotient.)
// Everything is compared in binary64, so the compiler cannot turn the
// reference into a binary32 division.
__device__ __forceinline__ bool nearest32(float got, double q) {
  const uint32_t b = __builtin_bit_cast(uint32_t, got);
  const double g = got;
  const double up = __builtin_bit_cast(float, b + 1u);
  const double dn = __builtin_bit_cast(float, b - 1u);
  const double d = fabs(g - q);
  return d < fabs(up - q) && d < fabs(dn - q);
}

__global__ __launch_bounds__(kProbeBlock) void sweep_kernel(int kind, uint32_t lo, uint32_t hi,
                                                            uint32_t per_thread,
                                                            uint32_t* counts) {
  __shared__ uint32_t part[kProbeBlock];
  const uint64_t first = (uint64_t)lo + ((uint64_t)blockIdx.x * kProbeBlock) * per_thread;
  uint32_t bad = 0;
  for (uint32_t k = 0; k < per_thread; ++k) {
    // consecutive threads take consecutive patterns
    const uint64_t b = first + (uint64_t)k * kProbeBlock + threadIdx.x;
    if (b >= hi) break;
    const float s = __builtin_bit_cast(float, (uint32_t)b);
    float got;
    double q;
    if (kind == 0) {
      got = recip_rn(s);
      q = 1.0 / (double)s;
    } else if (kind == 1) {
      got = scale_e4m3(s);
      q = (double)s / 448.0;
    } else {
      got = 1.0f / s;
      q = 1.0 / (double)s;
    }
    bad += nearest32(got, q) ? 0u : 1u;
  }
  part[threadIdx.x] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t sum = 0;
    for (int i = 0; i < kProbeBlock; ++i) sum += part[i];
    counts[blockIdx.x] = sum;
  }
}

__global__ __launch_bounds__(kProbeBlock) void recip_values_kernel(const float* s, float* r,
                                                                   float* sc, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
  if (i >= n) return;
  r[i] = recip_rn(s[i]);
  sc[i] = scale_e4m3(s[i]);
}

}  // namespace
}  // namespace qrw

using namespace qrw;

extern "C" int qrw_probe_copy_fused_traffic(const void* x, const void* w, const void* cos,
                                            const void* sin, uint8_t* q, float* scales,
                                            int64_t tokens, int64_t n, int wave_dependency,
                                            void* stream) {
  if (n != 4096 || tokens < 0 || tokens > (int64_t)0x7FFFFFFF) return QRW_ERR_SHAPE;
  if (tokens == 0) return QRW_OK;
  if (!x || !w || !cos || !sin || !q || !scales) return QRW_ERR_NULL;
  if (!al16(x) || !al16(w) || !al16(cos) || !al16(sin) || !al16(q)) return QRW_ERR_ALIGN;
  const dim3 grid((unsigned)((tokens + kProbeRows - 1) / kProbeRows));
  auto st = static_cast<hipStream_t>(stream);
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  const auto* cp = static_cast<const uint16_t*>(cos);
  const auto* sp = static_cast<const uint16_t*>(sin);
  if (wave_dependency)
    copy_fused_traffic_kernel<true><<<grid, kProbeBlock, 0, st>>>(xp, wp, cp, sp, q, scales, tokens);
  else
    copy_fused_traffic_kernel<false><<<grid, kProbeBlock, 0, st>>>(xp, wp, cp, sp, q, scales, tokens);
  return status_of(hipGetLastError());
}

extern "C" int qrw_probe_copy_qk_traffic(void* qkv, const void* q_weight, const void* k_weight,
                                         const void* cos, const void* sin, uint8_t* k_cache,
                                         uint8_t* v_cache, float* k_scales, float* v_scales,
                                         const int64_t* slots, int64_t num_slots, int64_t tokens,
                                         int kv, void* stream) {
  if (tokens < 0 || tokens > (int64_t)0x7FFFFFFF || (kv && num_slots < 0)) return QRW_ERR_SHAPE;
  if (tokens == 0) return QRW_OK;
  if (!qkv || !q_weight || !k_weight || !cos || !sin) return QRW_ERR_NULL;
  if (kv && (!k_cache || !v_cache || !k_scales || !v_scales || !slots)) return QRW_ERR_NULL;
  if (!al16(qkv) || !al16(q_weight) || !al16(k_weight) || !al16(cos) || !al16(sin))
    return QRW_ERR_ALIGN;
  if (kv && ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 7u))
    return QRW_ERR_ALIGN;
  const dim3 grid((unsigned)((tokens + kProbeRows - 1) / kProbeRows));
  auto st = static_cast<hipStream_t>(stream);
  auto* xp = static_cast<uint16_t*>(qkv);
  const auto* wqp = static_cast<const uint16_t*>(q_weight);
  const auto* wkp = static_cast<const uint16_t*>(k_weight);
  const auto* cp = static_cast<const uint16_t*>(cos);
  const auto* sp = static_cast<const uint16_t*>(sin);
  if (kv)
    copy_qk_traffic_kernel<true><<<grid, kProbeBlock, 0, st>>>(
        xp, wqp, wkp, cp, sp, k_cache, v_cache, k_scales, v_scales, slots, num_slots, tokens);
  else
    copy_qk_traffic_kernel<false><<<grid, kProbeBlock, 0, st>>>(
        xp, wqp, wkp, cp, sp, nullptr, nullptr, nullptr, nullptr, nullptr, 0, tokens);
  return status_of(hipGetLastError());
}

extern "C" int qrw_probe_empty(uint32_t* out, int64_t blocks, void* stream) {
  if (blocks < 0 || blocks > (int64_t)0x7FFFFFFF) return QRW_ERR_SHAPE;
  if (blocks == 0) return QRW_OK;
  if (!out) return QRW_ERR_NULL;
  empty_kernel<<<dim3((unsigned)blocks), kProbeBlock, 0, static_cast<hipStream_t>(stream)>>>(out);
  return status_of(hipGetLastError());
}

extern "C" int qrw_probe_fused_timeline(const void* x, const void* w, const void* cos,
                                        const void* sin, uint8_t* q, float* scales,
                                        int64_t tokens, float eps, uint64_t* stamps,
                                        void* stream) {
  if (tokens < 0 || tokens > (int64_t)0x7FFFFFFF) return QRW_ERR_SHAPE;
  if (tokens == 0) return QRW_OK;
  if (!x || !w || !cos || !sin || !q || !scales || !stamps) return QRW_ERR_NULL;
  if (!al16(x) || !al16(w) || !al16(cos) || !al16(sin) || !al16(q)) return QRW_ERR_ALIGN;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return QRW_ERR_VALUE;
  constexpr int R = kContigRows;
  const dim3 grid((unsigned)((tokens + R - 1) / R));
  fused_timeline_kernel<true><<<grid, kWave * R, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), cos, sin, q, scales,
      tokens, eps, stamps);
  return status_of(hipGetLastError());
}

extern "C" int qrw_probe_sweep(int kind, uint32_t lo_bits, uint32_t hi_bits, uint32_t per_thread,
                               uint32_t* counts, int64_t blocks, void* stream) {
  if (kind < 0 || kind > 2) return QRW_ERR_VALUE;
  if (!(lo_bits < hi_bits) || hi_bits > 0x7F800000u) return QRW_ERR_SHAPE;
  if (per_thread < 1 || per_thread > 4096) return QRW_ERR_SHAPE;
  const uint64_t per_block = (uint64_t)kProbeBlock * per_thread;
  const uint64_t need = ((uint64_t)(hi_bits - lo_bits) + per_block - 1) / per_block;
  if (blocks != (int64_t)need) return QRW_ERR_SHAPE;
  if (!counts) return QRW_ERR_NULL;
  sweep_kernel<<<dim3((unsigned)blocks), kProbeBlock, 0, static_cast<hipStream_t>(stream)>>>(
      kind, lo_bits, hi_bits, per_thread, counts);
  return status_of(hipGetLastError());
}

extern "C" int qrw_probe_recip_values(const float* s, float* out_recip, float* out_scale,
                                      int64_t n, void* stream) {
  if (n < 0 || n > ((int64_t)0x7FFFFFFF) * kProbeBlock) return QRW_ERR_SHAPE;
  if (n == 0) return QRW_OK;
  if (!s || !out_recip || !out_scale) return QRW_ERR_NULL;
  const dim3 grid((unsigned)((n + kProbeBlock - 1) / kProbeBlock));
  recip_values_kernel<<<grid, kProbeBlock, 0, static_cast<hipStream_t>(stream)>>>(
      s, out_recip, out_scale, n);
  return status_of(hipGetLastError());
}
