// qrw_norm.hip -- one-pass RMSNorm and LayerNorm row kernels (gfx950).
//
// Definitions: "TileLang tutorial, ch. 13", s3.2.1 (reference RMSNorm and
// LayerNorm), with the register-resident design of s3.2.3: each row is read
// from HBM once and stays in VGPRs while its statistics are reduced.
//
// Mapping: one wave64 per row, four rows per 256-thread workgroup.  Lane l
// owns granules l, l+64, l+128, ... (GPL of them), so each load instruction
// of a wave covers 1 KiB of contiguous row.  Row statistics: eight per-lane
// partial sums (one per element slot of a granule, a shallow serial chain),
// a fixed pairwise tree, then the wave64 DPP reduction.
//
// Cache hints (measured on MI355X at 4096 x 4096): the rows are touched once
// per launch, so outputs are written with non-temporal stores; LayerNorm also
// reads x non-temporally, RMSNorm reads it normally (faster there).
//
// Arithmetic (binary32, one final rounding):
//   RMSNorm   y = (x * w) * rstd      x*w is exact in binary32 for 16-bit x, w
//   LayerNorm y = fma(((x - mu0) - r) * rstd, gamma, beta), mu = mu0 + r
#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

template <typename T, int GPL, bool FULL>
__global__ __launch_bounds__(kBlock) void rmsnorm_kernel(const uint16_t* x,
                                                         const uint16_t* __restrict__ w,
                                                         uint16_t* y, int64_t rows, int ng,
                                                         int64_t xs, int64_t ys, float n_f,
                                                         float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;

  u32x4 raw[GPL];
  u32x4 wr[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16(xr + 8 * gi);
  }
  if (w) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave + lane;
      wr[g] = (u32x4){0u, 0u, 0u, 0u};
      if (FULL || gi < ng) wr[g] = ld16(w + 8 * gi);
    }
  }

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(v[k], v[k], acc[k]);
  }
  const float ss = wave_sum(tree8(acc));
  const float rstd = 1.0f / sqrtf(ss / n_f + eps);

#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    if (FULL || gi < ng) {
      float v[8];
      widen8<T>(raw[g], v);
      if (w) {
        float wv[8];
        widen8<T>(wr[g], wv);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (v[k] * wv[k]) * rstd;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] * rstd;
      }
      st16_stream(yr + 8 * gi, narrow8<T>(v));
    }
  }
}

template <typename T, int GPL, bool FULL>
__global__ __launch_bounds__(kBlock) void layernorm_kernel(const uint16_t* x,
                                                           const uint16_t* __restrict__ gam,
                                                           const uint16_t* __restrict__ bet,
                                                           uint16_t* y, int64_t rows, int ng,
                                                           int64_t xs, int64_t ys, float n_f,
                                                           float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;

  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16_stream(xr + 8 * gi);
  }

  // Mean in two parts: mu0 is the binary32 mean; the mean r of the residuals
  // x - mu0 comes out of the same register pass as the centred second moment,
  // so the centring (x - mu0) - r carries mu0's rounding error.  Outputs that
  // are a near-cancellation of (x - mu) * rstd * gamma and beta then keep
  // their accuracy.
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += v[k];
  }
  const float mu0 = wave_sum(tree8(acc)) / n_f;

  // biased variance around the mean, from the registers (second pass over VGPRs)
  float acc1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float acc2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    if (FULL || gi < ng) {
      float v[8];
      widen8<T>(raw[g], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float d = v[k] - mu0;
        acc1[k] += d;
        acc2[k] = fmaf(d, d, acc2[k]);
      }
    }
  }
  const float r = wave_sum(tree8(acc1)) / n_f;
  const float m2 = wave_sum(tree8(acc2)) / n_f;
  const float var = fmaxf(fmaf(-r, r, m2), 0.0f);  // mean((x - mu0 - r)^2)
  const float rstd = 1.0f / sqrtf(var + eps);

#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    if (FULL || gi < ng) {
      float v[8], gv[8], bv[8];
      widen8<T>(raw[g], v);
      if (gam) {
        widen8<T>(ld16(gam + 8 * gi), gv);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) gv[k] = 1.0f;
      }
      if (bet) {
        widen8<T>(ld16(bet + 8 * gi), bv);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) bv[k] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = fmaf(((v[k] - mu0) - r) * rstd, gv[k], bv[k]);
      st16_stream(yr + 8 * gi, narrow8<T>(v));
    }
  }
}

// ------------------------------------------------------------------ launch
namespace {

int granules_per_lane(int ng) {
  return ng <= 64 ? 1 : ng <= 128 ? 2 : ng <= 256 ? 4 : ng <= 512 ? 8 : 16;
}

}  // namespace

#define QRW_NORM_DISPATCH(KERNEL, T, gpl, full, grid, stream, ...)                       \
  do {                                                                                   \
    switch (gpl) {                                                                       \
      case 1:                                                                            \
        if (full) KERNEL<T, 1, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);          \
        else KERNEL<T, 1, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);             \
        break;                                                                           \
      case 2:                                                                            \
        if (full) KERNEL<T, 2, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);          \
        else KERNEL<T, 2, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);             \
        break;                                                                           \
      case 4:                                                                            \
        if (full) KERNEL<T, 4, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);          \
        else KERNEL<T, 4, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);             \
        break;                                                                           \
      case 8:                                                                            \
        if (full) KERNEL<T, 8, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);          \
        else KERNEL<T, 8, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);             \
        break;                                                                           \
      default:                                                                           \
        if (full) KERNEL<T, 16, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);         \
        else KERNEL<T, 16, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);            \
        break;                                                                           \
    }                                                                                    \
  } while (0)

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int64_t n,
                          int64_t xs, int64_t ys, int dtype, float eps, hipStream_t stream) {
  const int ng = (int)(n / 8);
  const int gpl = granules_per_lane(ng);
  const bool full = ng == gpl * kWave;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  auto* yp = static_cast<uint16_t*>(y);
  if (dtype == 1) {
    QRW_NORM_DISPATCH(rmsnorm_kernel, F16, gpl, full, grid, stream, xp, wp, yp, rows, ng, xs, ys,
                      (float)n, eps);
  } else {
    QRW_NORM_DISPATCH(rmsnorm_kernel, BF16, gpl, full, grid, stream, xp, wp, yp, rows, ng, xs,
                      ys, (float)n, eps);
  }
  return hipGetLastError();
}

hipError_t launch_layernorm(const void* x, const void* g, const void* b, void* y, int64_t rows,
                            int64_t n, int64_t xs, int64_t ys, int dtype, float eps,
                            hipStream_t stream) {
  const int ng = (int)(n / 8);
  const int gpl = granules_per_lane(ng);
  const bool full = ng == gpl * kWave;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* gp = static_cast<const uint16_t*>(g);
  const auto* bp = static_cast<const uint16_t*>(b);
  auto* yp = static_cast<uint16_t*>(y);
  if (dtype == 1) {
    QRW_NORM_DISPATCH(layernorm_kernel, F16, gpl, full, grid, stream, xp, gp, bp, yp, rows, ng,
                      xs, ys, (float)n, eps);
  } else {
    QRW_NORM_DISPATCH(layernorm_kernel, BF16, gpl, full, grid, stream, xp, gp, bp, yp, rows, ng,
                      xs, ys, (float)n, eps);
  }
  return hipGetLastError();
}

}  // namespace qrw
