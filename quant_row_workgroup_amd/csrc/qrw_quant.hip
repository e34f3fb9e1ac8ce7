// qrw_quant.hip -- activation quantisation to OCP E4M3FN, one scale per token
// or per group of consecutive channels (gfx950).
//
// Definition: "TileLang tutorial, ch. 13", s3.1.5 (the per-token / per-group
// cast): amax over the group -> scale = max(amax, 1e-4) / fp8_max -> codes of
// clamp(x / scale, -fp8_max, fp8_max), fp8_max = 448 for E4M3FN.
//
// Mapping: one wave64 per row; lane l owns granules l, l+64, ... (GPL of
// them), so each load instruction covers 1 KiB of contiguous row and each
// code store 512 B.  A group of `group` channels is group/8 consecutive lanes
// of one load instruction; its amax is reduced with DPP inside the lane group
// (quad permutes, half-row and row mirrors) or with the LDS crossbar for 32
// lanes, and for a whole-row group with the wave reduction.  x is read and the
// codes are written with non-temporal hints (measured faster on MI355X).
//
// The code of x is the E4M3 rounding of the binary32 quotient x / scale, as
// the page's cast computes it in float32.  The quotient is formed correctly
// rounded without a division per element (Markstein's correction): with
// y = RN(1/scale) once per group, q = RN(x*y), r = x - q*scale (exact, one
// fma), RN(q + r*y) is RN(x/scale).  |x| <= amax makes the largest quotient
// at most 448 * (1 + 2^-23) < 464, so the conversion stays finite and the
// clamp cannot act.
#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

template <typename T, int GPL, bool FULL, int L>
__global__ __launch_bounds__(kBlock) void act_quant_group_kernel(const uint16_t* x, uint8_t* q,
                                                                 float* scales, int64_t rows,
                                                                 int ng, int64_t xs, int64_t qs,
                                                                 int64_t groups) {
  // When a whole row has at most 64 groups (GPL <= L), lane j collects the
  // scale of group j (from any lane of that group, by a lane permute) and the
  // row's scales leave in one contiguous store instead of one store per group.
  constexpr bool kGather = FULL && GPL <= L;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * xs;
  uint8_t* qr = q + row * qs;
  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16_stream(xr + 8 * gi);
  }
  float mine = 0.0f;
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    float v[8];
    widen8<T>(raw[g], v);
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) m = fmaxf(m, fmaxf(fabsf(v[e]), fabsf(v[e + 1])));
    const float am = fmaxf(group_max<L>(m), 1e-4f);  // groups never straddle the row end
    const float scale = scale_e4m3(am);
    if constexpr (kGather) {
      // groups g*(64/L) .. of this step sit in lane blocks of L; lane j takes
      // group j = g*(64/L) + q from lane q*L
      constexpr int kPer = kWave / L;
      const int src = (lane % kPer) * L;
      const float got = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(src * 4, __builtin_bit_cast(int, scale)));
      if (lane / kPer == g) mine = got;
    }
    if (FULL || gi < ng) {
      const float y = recip_rn(scale);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], scale, y);
      st8_stream(qr + 8 * gi, fp8x8(v));
      if (!kGather && (lane & (L - 1)) == 0) scales[row * groups + gi / L] = scale;
    }
  }
  if constexpr (kGather) {
    if (lane < GPL * (kWave / L)) scales[row * groups + lane] = mine;
  }
}

// One scale per row.
template <typename T, int GPL, bool FULL>
__global__ __launch_bounds__(kBlock) void act_quant_token_kernel(const uint16_t* x, uint8_t* q,
                                                                 float* scales, int64_t rows,
                                                                 int ng, int64_t xs,
                                                                 int64_t qs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * xs;
  uint8_t* qr = q + row * qs;
  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16_stream(xr + 8 * gi);
  }
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      m[e >> 1] = fmaxf(m[e >> 1], fmaxf(fabsf(v[e]), fabsf(v[e + 1])));
  }
  const float am = fmaxf(wave_max(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]))), 1e-4f);
  const float scale = scale_e4m3(am);
  const float y = recip_rn(scale);
  if (lane == 0) scales[row] = scale;
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    if (FULL || gi < ng) {
      float v[8];
      widen8<T>(raw[g], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], scale, y);
      st8_stream(qr + 8 * gi, fp8x8(v));
    }
  }
}

// ------------------------------------------------------------------ launch
namespace {

int quant_gpl(int ng) { return ng <= 64 ? 1 : ng <= 128 ? 2 : ng <= 256 ? 4 : ng <= 512 ? 8 : 16; }

template <typename T, int GPL, bool FULL>
void group_go(int lanes, dim3 grid, hipStream_t st, const uint16_t* x, uint8_t* q, float* sc,
              int64_t rows, int ng, int64_t xs, int64_t qs, int64_t groups) {
  switch (lanes) {
    case 1: act_quant_group_kernel<T, GPL, FULL, 1><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
    case 2: act_quant_group_kernel<T, GPL, FULL, 2><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
    case 4: act_quant_group_kernel<T, GPL, FULL, 4><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
    case 8: act_quant_group_kernel<T, GPL, FULL, 8><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
    case 16: act_quant_group_kernel<T, GPL, FULL, 16><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
    case 32: act_quant_group_kernel<T, GPL, FULL, 32><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
    default: act_quant_group_kernel<T, GPL, FULL, 64><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups); break;
  }
}

template <typename T, int GPL, bool FULL>
void quant_go(int64_t group, int64_t n, dim3 grid, hipStream_t st, const uint16_t* x, uint8_t* q,
              float* sc, int64_t rows, int ng, int64_t xs, int64_t qs) {
  if (group == n)
    act_quant_token_kernel<T, GPL, FULL><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs);
  else
    group_go<T, GPL, FULL>((int)(group / 8), grid, st, x, q, sc, rows, ng, xs, qs, n / group);
}

template <typename T>
void quant_dispatch(int64_t group, int64_t n, dim3 grid, hipStream_t st, const uint16_t* x,
                    uint8_t* q, float* sc, int64_t rows, int64_t xs, int64_t qs) {
  const int ng = (int)(n / 8);
  const int gpl = quant_gpl(ng);
  const bool full = ng == gpl * kWave;
  switch (gpl) {
    case 1: full ? quant_go<T, 1, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 1, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    case 2: full ? quant_go<T, 2, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 2, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    case 4: full ? quant_go<T, 4, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 4, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    case 8: full ? quant_go<T, 8, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 8, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    default: full ? quant_go<T, 16, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 16, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
  }
}

}  // namespace

hipError_t launch_act_quant_fp8(const void* x, uint8_t* q, float* scales, int64_t rows,
                                int64_t n, int64_t group, int64_t xs, int64_t qs, int dtype,
                                hipStream_t stream) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto* xp = static_cast<const uint16_t*>(x);
  if (dtype == 1)
    quant_dispatch<F16>(group, n, grid, stream, xp, q, scales, rows, xs, qs);
  else
    quant_dispatch<BF16>(group, n, grid, stream, xp, q, scales, rows, xs, qs);
  return hipGetLastError();
}

}  // namespace qrw
