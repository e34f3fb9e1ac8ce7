// qrw_norm.hip -- one-pass RMSNorm and LayerNorm row kernels (gfx950).
//
// Definitions: "TileLang tutorial, ch. 13", s3.2.1 (reference RMSNorm and
// LayerNorm), with the register-resident design of s3.2.3: each row is read
// from HBM once and stays in VGPRs while its statistics are reduced.
//
// Mapping: one wave64 per row, four rows per 256-thread workgroup.  Lane l
// owns granules l, l+64, l+128, ... (GPL of them), so each load instruction
// of a wave covers 1 KiB of contiguous row.  Row statistics: eight per-lane
// partial sums (a shallow serial chain each), a fixed pairwise tree, then the
// wave64 DPP reduction.  The one-wave RMSNorm forms its sum of squares on the
// packed 16-bit pairs with v_dot2 (the products are exact in binary32); the
// other kernels widen and use fma.
//
// Cache hints (measured on MI355X at 4096 x 4096): the rows are touched once
// per launch, so outputs are written with non-temporal stores; LayerNorm also
// reads x non-temporally, RMSNorm reads it normally (faster there).
//
// Arithmetic (binary32, one final rounding):
//   RMSNorm   y = (x * w) * rstd      x*w is exact in binary32 for 16-bit x, w
//   LayerNorm y = fma(((x - mu0) - r) * rstd, gamma, beta), mu = mu0 + r
#include <algorithm>

#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

// A row whose length is not a multiple of 8 ends in one partial granule,
// index nfull = n >> 3 (TAIL).  Every other granule is whole and takes a full
// 16-byte access under a plain `gi < nfull` mask; the partial one is held in
// a register pair of its own by the thread whose granule sequence it ends, so
// that thread's accumulation order is the same as if it sat in the array.
// Whole granule gi of a row, or zeros where gi >= nfull (requires nfull >= 1).
// Branch-free: a masked lane re-reads the row's last whole granule, which its
// neighbours load anyway, and drops it.  (A branch per granule makes the
// compiler copy every live register at each join.)
template <bool STREAM>
__device__ __forceinline__ u32x4 ld_masked(const uint16_t* p, int gi, int nfull) {
  const bool in = gi < nfull;
  const uint16_t* q = p + 8 * (in ? gi : nfull - 1);
  const u32x4 v = STREAM ? ld16_stream(q) : ld16(q);
  return in ? v : (u32x4){0u, 0u, 0u, 0u};
}

template <bool TAIL>
__device__ __forceinline__ u32x4 ld_tail(const uint16_t* p, bool mine, int nfull, int n) {
  if (TAIL && mine) return ld_partial(p + 8 * nfull, n & 7);
  return (u32x4){0u, 0u, 0u, 0u};
}

// Occupancy floor (waves per SIMD) of the one-wave kernels: 4 (<= 128 VGPRs)
// up to 8 granules per lane, 2 for 16 (the row alone is 64 VGPRs).  A launch
// of 4096 rows is 4 waves per SIMD, so below 4 a quarter of the rows wait for
// a second round.  Without a floor the compiler's choice swings between ~80
// and ~250 VGPRs from one instance to the next.  The row-block kernels ask for
// 8 at 4 granules per thread (7 for ragged LayerNorm, which spills at 8) and
// 4 at 8 granules.
template <int GPL, bool TAIL>
constexpr int kNormWaves = GPL <= 8 ? 4 : 2;

// HAS_W: w is given.  Taking it as a template parameter rather than testing
// the pointer keeps the weighted and unweighted paths from joining before the
// row's sum: at such a join the compiler's wait for x counted the weight loads
// as well, so the sum waited for the (cold, every-row) weight.  Measured on
// MI355X (bf16/f16, 1 GiB of rotating buffers): 4096 x 4096 1.10x as fast,
// 256 x 1024 1.05x, 16384 x 512 1.07x, 4096 x 8192 1.07x, 8192 x 1024-2048
// 1.01-1.02x; 4096 x 4095 and 1024 x 4096 0.99x.
// LATE_W: w is read at output time, after the row's sum, as the ragged form
// always does.  With at least 4 workgroups per CU (then every wave of the
// launch is resident at once and all of them would request w with x) that
// measured 0.99-1.08x as fast (4096 x 4096 f16 1.06x, 65536 x 128 1.08x,
// 4096 x 1000 1.05x); with fewer, where the extra round trip is exposed,
// 0.90x (1024 x 4096).
template <typename T, int GPL, bool FULL, bool TAIL, bool HAS_W, bool LATE_W>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kNormWaves<GPL, TAIL>))) void rmsnorm_kernel(const uint16_t* x,
                                                         const uint16_t* __restrict__ w,
                                                         uint16_t* y, int64_t rows, int nfull,
                                                         int n, int64_t xs, int64_t ys,
                                                         float n_f, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  const bool mine = TAIL && lane == (nfull & (kWave - 1));

  u32x4 raw[GPL];
  u32x4 wr[GPL];
  // a row with no whole granule (n < 8) needs GPL == 1; at 2 or more granules
  // per lane the test is a constant, which keeps the loads free of a branch
  // (4096 x 4095 bf16: 12.0 against 12.5 us with the run-time test)
  const bool any = FULL || GPL > 1 || nfull > 0;  // wave-uniform
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (any) raw[g] = FULL ? ld16(xr + 8 * gi) : ld_masked<false>(xr, gi, nfull);
  }
  const u32x4 xt = ld_tail<TAIL>(xr, mine, nfull, n);
  // The weights are loaded with x, except in the ragged form, which reads
  // them at output time (measured faster there: 12.9 against 14.4 us on
  // 4096 x 4095 bf16), and with LATE_W.
  constexpr bool kPreW = !TAIL && !LATE_W;
  if (kPreW && HAS_W) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave + lane;
      wr[g] = (u32x4){0u, 0u, 0u, 0u};
      if (any) wr[g] = FULL ? ld16(w + 8 * gi) : ld_masked<false>(w, gi, nfull);
    }
  }

  // sum of squares on the packed pairs (v_dot2: the 16-bit products are exact)
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[(4 * g + k) & 7] = sumsq2(T{}, raw[g][k], acc[(4 * g + k) & 7]);
  }
  if (TAIL) {  // the partial granule ends its lane's sequence
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[(4 * GPL + k) & 7] = sumsq2(T{}, xt[k], acc[(4 * GPL + k) & 7]);
  }
  const float ss = wave_sum(tree8(acc));
  const float rstd = 1.0f / sqrtf(ss / n_f + eps);

  auto finish = [&](u32x4 xg, u32x4 wg) {
    float v[8];
    widen8<T>(xg, v);
    if (HAS_W) {
      float wv[8];
      widen8<T>(wg, wv);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (v[k] * wv[k]) * rstd;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = v[k] * rstd;
    }
    return narrow8<T>(v);
  };
  if (!kPreW && HAS_W) {  // late weights
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave + lane;
      if (FULL || gi < nfull) st16_stream(yr + 8 * gi, finish(raw[g], ld16(w + 8 * gi)));
    }
  } else {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave + lane;
      if (FULL || gi < nfull)
        st16_stream(yr + 8 * gi, finish(raw[g], HAS_W ? wr[g] : (u32x4){0u, 0u, 0u, 0u}));
    }
  }
  if (mine) st_partial(yr + 8 * nfull, finish(xt, ld_tail<TAIL>(w, HAS_W, nfull, n)), n & 7);
}

// The weight cases in the dispatch macro's four-parameter form.
template <typename T, int GPL, bool FULL, bool TAIL>
constexpr auto rmsnorm_w_kernel = rmsnorm_kernel<T, GPL, FULL, TAIL, true, false>;
template <typename T, int GPL, bool FULL, bool TAIL>
constexpr auto rmsnorm_wlate_kernel = rmsnorm_kernel<T, GPL, FULL, TAIL, true, true>;
template <typename T, int GPL, bool FULL, bool TAIL>
constexpr auto rmsnorm_now_kernel = rmsnorm_kernel<T, GPL, FULL, TAIL, false, false>;

// LayerNorm's centred pass over one granule: the first cnt elements are
// centred on mu0 and accumulated; padding elements are not centred.
__device__ __forceinline__ void centred_moments(const float (&v)[8], int cnt, float mu0,
                                                float (&acc1)[8], float (&acc2)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float d = k < cnt ? v[k] - mu0 : 0.0f;
    acc1[k] += d;
    acc2[k] = fmaf(d, d, acc2[k]);
  }
}

// y = ((x - mu0) - r) * rstd * gamma + beta for one granule; absent gamma is
// 1, absent beta 0.
template <typename T>
__device__ __forceinline__ u32x4 layernorm_out(u32x4 xg, u32x4 gg, u32x4 bg, bool has_g,
                                               bool has_b, float mu0, float r, float rstd) {
  float v[8], gv[8], bv[8];
  widen8<T>(xg, v);
  widen8<T>(gg, gv);
  widen8<T>(bg, bv);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    v[k] = fmaf(((v[k] - mu0) - r) * rstd, has_g ? gv[k] : 1.0f, has_b ? bv[k] : 0.0f);
  return narrow8<T>(v);
}

template <typename T, int GPL, bool FULL, bool TAIL>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kNormWaves<GPL, TAIL>))) void layernorm_kernel(const uint16_t* x,
                                                           const uint16_t* __restrict__ gam,
                                                           const uint16_t* __restrict__ bet,
                                                           uint16_t* y, int64_t rows, int nfull,
                                                           int n, int64_t xs, int64_t ys,
                                                           float n_f, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  const bool mine = TAIL && lane == (nfull & (kWave - 1));

  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < nfull) raw[g] = ld16_stream(xr + 8 * gi);
  }
  const u32x4 xt = ld_tail<TAIL>(xr, mine, nfull, n);

  // Mean in two parts: mu0 is the binary32 mean; the mean r of the residuals
  // x - mu0 comes out of the same register pass as the centred second moment,
  // so the centring (x - mu0) - r carries mu0's rounding error.  Outputs that
  // are a near-cancellation of (x - mu) * rstd * gamma and beta then keep
  // their accuracy.
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL + (TAIL ? 1 : 0); ++g) {
    float v[8];
    widen8<T>(g < GPL ? raw[g] : xt, v);
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
    float v[8];
    widen8<T>(raw[g], v);
    centred_moments(v, FULL || gi < nfull ? 8 : 0, mu0, acc1, acc2);
  }
  if (mine) {
    float v[8];
    widen8<T>(xt, v);
    centred_moments(v, n & 7, mu0, acc1, acc2);
  }
  const float r = wave_sum(tree8(acc1)) / n_f;
  const float m2 = wave_sum(tree8(acc2)) / n_f;
  const float var = fmaxf(fmaf(-r, r, m2), 0.0f);  // mean((x - mu0 - r)^2)
  const float rstd = 1.0f / sqrtf(var + eps);

  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  if (gam && bet) {
    // the affine case without a test per granule, so that the gamma/beta
    // loads of later granules can be issued ahead of earlier granules' math
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave + lane;
      if (FULL || gi < nfull)
        st16_stream(yr + 8 * gi, layernorm_out<T>(raw[g], ld16(gam + 8 * gi),
                                                  ld16(bet + 8 * gi), true, true, mu0, r, rstd));
    }
  } else {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave + lane;
      if (FULL || gi < nfull)
        st16_stream(yr + 8 * gi, layernorm_out<T>(raw[g], gam ? ld16(gam + 8 * gi) : zero,
                                                  bet ? ld16(bet + 8 * gi) : zero, gam != nullptr,
                                                  bet != nullptr, mu0, r, rstd));
    }
  }
  if (mine)
    st_partial(yr + 8 * nfull,
               layernorm_out<T>(xt, ld_tail<TAIL>(gam, gam != nullptr, nfull, n),
                                ld_tail<TAIL>(bet, bet != nullptr, nfull, n), gam != nullptr,
                                bet != nullptr, mu0, r, rstd),
               n & 7);
}

// ------------------------------------------------------ rows of many waves
// Rows longer than one wave holds (8192 elements) stay register-resident in a
// workgroup of W waves (s3.2.3's design with a wider tile): thread t owns
// granules t, t + 64W, t + 128W, ...  Row statistics: each wave's DPP sum is
// left in an LDS slot per wave, and after one barrier every lane adds the W
// slots in a fixed pairwise order (s3.2's two-level reduction: in-thread, then
// across threads, with a per-wave workspace).

// Sum of v over the workgroup's W waves; every lane gets the same value.
template <int W>
__device__ __forceinline__ float block_sum(float v, float* slot) {
  const float ws = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) slot[threadIdx.x >> 6] = ws;
  __syncthreads();
  float s[W];
#pragma unroll
  for (int i = 0; i < W; ++i) s[i] = slot[i];
#pragma unroll
  for (int h = W / 2; h >= 1; h /= 2)
#pragma unroll
    for (int i = 0; i < h; ++i) s[i] += s[i + h];
  return s[0];
}

// RMSNorm output of one granule: (x * w) * rstd, or x * rstd without weights.
template <typename T>
__device__ __forceinline__ u32x4 rmsnorm_granule(u32x4 xg, u32x4 wg, bool has_w, float rstd) {
  float v[8];
  widen8<T>(xg, v);
  if (has_w) {
    float wv[8];
    widen8<T>(wg, wv);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (v[k] * wv[k]) * rstd;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = v[k] * rstd;
  }
  return narrow8<T>(v);
}

// EARLY (w given): the weight is requested right after x instead of at
// output time, for launches of at most 8 waves per CU, where a wave's latency
// is what shows (the one-wave LayerNorm's rule); occupancy does not matter
// there, so these instances may use up to 256 VGPRs.
template <typename T, int W, int GPL, bool TAIL, bool EARLY>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(EARLY ? 2 : GPL <= 4 ? 8 : 4))) void rmsnorm_rowblock_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, uint16_t* y, int nfull, int n, int64_t xs,
    int64_t ys, float n_f, float eps) {
  __shared__ float slot[W];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  const bool mine = TAIL && t == nfull % (kWave * W);
  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave * W + t;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (gi < nfull) raw[g] = ld16(xr + 8 * gi);
  }
  const u32x4 xt = ld_tail<TAIL>(xr, mine, nfull, n);
  u32x4 wr[GPL];
  if (EARLY) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      wr[g] = (u32x4){0u, 0u, 0u, 0u};
      if (gi < nfull) wr[g] = ld16(w + 8 * gi);
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL + (TAIL ? 1 : 0); ++g) {
    float v[8];
    widen8<T>(g < GPL ? raw[g] : xt, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(v[k], v[k], acc[k]);
  }
  const float ss = block_sum<W>(tree8(acc), slot);
  const float rstd = 1.0f / sqrtf(ss / n_f + eps);
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  if (EARLY) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      if (gi < nfull) st16_stream(yr + 8 * gi, rmsnorm_granule<T>(raw[g], wr[g], true, rstd));
    }
  } else if (w) {  // no test per granule, so later weight loads run ahead of the math
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      if (gi < nfull) st16_stream(yr + 8 * gi, rmsnorm_granule<T>(raw[g], ld16(w + 8 * gi), true, rstd));
    }
  } else {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      if (gi < nfull) st16_stream(yr + 8 * gi, rmsnorm_granule<T>(raw[g], zero, false, rstd));
    }
  }
  if (mine)
    st_partial(yr + 8 * nfull,
               rmsnorm_granule<T>(xt, w ? ld_partial(w + 8 * nfull, n & 7) : zero,
                                  w != nullptr, rstd),
               n & 7);
}

// The two weight placements in the dispatch macro's four-parameter form.
template <typename T, int W, int GPL, bool TAIL>
constexpr auto rmsnorm_rowblock_late = rmsnorm_rowblock_kernel<T, W, GPL, TAIL, false>;
template <typename T, int W, int GPL, bool TAIL>
constexpr auto rmsnorm_rowblock_early = rmsnorm_rowblock_kernel<T, W, GPL, TAIL, true>;

// Row-block shape for kOneWaveGranules < ng <= kResidentGranules: gpt granules
// per thread (4, or 8 for rows beyond 4 granules x max_waves waves), and the
// smallest power of two in [2, 16] of waves whose threads hold the row.  At 4
// granules (16 VGPRs of row data) the kernels run at up to 8 waves per SIMD;
// at 8 (32 VGPRs) a 1024-thread workgroup stays within 128 VGPRs per lane.
// Measured on MI355X (bf16): RMSNorm 2048 x 16384 25.3 against 27.3 us and
// 1024 x 32768 26.6 against 27.3 us at 4; LayerNorm, whose three block sums
// cost more at 16 waves, takes 4 only up to 8 waves (2048 x 16384: 27.7
// against 28.2 us; 1024 x 32768 at 16 waves x 4: 29.5 against 28.2 us).
struct BlockShape {
  int waves, gpt;
};
constexpr int kRmsMaxWavesAt4 = 16, kLnMaxWavesAt4 = 8;  // the two operators' choices above
inline BlockShape block_shape(int ng, int max_waves_at_4) {
  const int gpt = ng <= max_waves_at_4 * kWave * 4 ? 4 : 8;
  int w = 2;
  while (w < 16 && w * kWave * gpt < ng) w *= 2;
  return {w, gpt};
}

// ------------------------------------------- rows of many waves, pipelined
// Rows of exactly 8 granules per thread of W = 4, 8 or 16 waves (n = 16384,
// 32768 or 65536 elements), where the grid is only as large as the GPU holds
// at once.  Each workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x, ...
// and loads its next row while it finishes the current one, so that its reads
// overlap its own writes instead of every resident row loading and then every
// one storing in lock step.  The per-row constants (RMSNorm's w, LayerNorm's
// gamma and beta) are loaded once per workgroup, and x is read non-temporally.
//
// Which kernel takes a row depends on how many rows share the launch, so the
// pipelined kernels reproduce the row-block kernel's sums bit for bit, and a
// row's output is the same in any batch.  LayerNorm's row-block kernel has
// the same shape on these rows.  RMSNorm's gives each of S * W waves' threads
// 8 / S granules (S = 2 at n = 16384 and 32768): thread t here holds the
// granules of its threads t + 64W*h, h < S, keeps S partial sums, and
// block_sum_split adds the S * W wave sums in block_sum's order.
//
// Measured on MI355X against the one-row-per-workgroup kernel (bf16, 8 or more
// rotating buffer sets of at least 1 GiB in all), by rows per resident
// workgroup: RMSNorm from 1.5 to 4 was 1.00-1.17x as fast (1024 x 32768 23.8
// against 25.4 us, 768 x 32768 17.0 against 19.8, 512 x 65536 23.0 against
// 25.3), at 1 or less mostly slower (512 x 32768 0.91x, 1024 x 16384 0.83x: a
// workgroup then holds one row with fewer waves than the row-block kernel), at
// 8 0.99x; rows with masked granules (1024 x 32760, 4096 x 8200, 8192 x 12288)
// were 2-4% slower.  So both operators take whole rows, from 1.5 to 4 rows per
// resident workgroup.
constexpr int kRowpipeGpl = 8;
constexpr int kRowpipeMaxRowsPerBlock = 4;

template <typename T>
constexpr uint32_t kOnePair = std::is_same<T, BF16>::value ? 0x3F803F80u : 0x3C003C00u;

// block_sum<S * W> of a workgroup of S * W waves, computed by W waves whose
// thread t (of wave i) holds in v[h] the partial sum of that workgroup's
// thread t + 64W*h: the wave sums go to slots h*W + i, and after one barrier
// the S * W slots are added in block_sum's pairwise order.
template <int W, int S>
__device__ __forceinline__ float block_sum_split(const float (&v)[S], float* slot) {
  float ws[S];
#pragma unroll
  for (int h = 0; h < S; ++h) ws[h] = wave_sum(v[h]);
  if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
    for (int h = 0; h < S; ++h) slot[h * W + (threadIdx.x >> 6)] = ws[h];
  }
  __syncthreads();
  float s[S * W];
#pragma unroll
  for (int i = 0; i < S * W; ++i) s[i] = slot[i];
#pragma unroll
  for (int h = S * W / 2; h >= 1; h /= 2)
#pragma unroll
    for (int i = 0; i < h; ++i) s[i] += s[i + h];
  return s[0];
}

// LayerNorm's statistics on rows of 8 whole granules per thread: each
// thread's mean m and centred sum of squares q over its own c elements, merged pairwise by Chan, Golub and LeVeque's update for two
// halves of equal count (the union's mean is the mean of the two means, and
// q gains d^2 c / 2 for d the difference of the means), across the lanes of
// a wave and then across the waves in block_sum's order, through one
// barrier.  Every step is symmetric in the two halves (d changes sign
// exactly, and no product is left for the compiler to contract), so both
// partners of an exchange hold the same bits.
__device__ __forceinline__ void chan_merge(float& m, float& q, float mo, float qo, float half_c) {
  const float d = mo - m;
  m = 0.5f * (m + mo);
  q = fmaf(d * d, half_c, q + qo);
}

// The merge over a wave's 64 lanes, each holding c elements, in wave_sum's
// pairing; every lane gets the result.
__device__ __forceinline__ void wave_chan(float& m, float& q, float c) {
  chan_merge(m, q, dpp<kDppXor1>(m), dpp<kDppXor1>(q), 0.5f * c);
  chan_merge(m, q, dpp<kDppXor2>(m), dpp<kDppXor2>(q), c);
  chan_merge(m, q, dpp<kDppHalfMirror>(m), dpp<kDppHalfMirror>(q), 2.0f * c);
  chan_merge(m, q, dpp<kDppMirror>(m), dpp<kDppMirror>(q), 4.0f * c);
  float m0 = lane_value(m, 0), q0 = lane_value(q, 0);
  float m2 = lane_value(m, 32), q2 = lane_value(q, 32);
  chan_merge(m0, q0, lane_value(m, 16), lane_value(q, 16), 8.0f * c);
  chan_merge(m2, q2, lane_value(m, 48), lane_value(q, 48), 8.0f * c);
  chan_merge(m0, q0, m2, q2, 16.0f * c);
  m = m0;
  q = q0;
}

// The merge over a workgroup of W waves whose threads hold statistics over
// c elements each, through slot (2 * W floats) and one barrier.  Returns the
// row's mean and its centred sum of squares.
template <int W>
__device__ __forceinline__ void block_chan(float m, float q, float c, float* slot, float& mean,
                                           float& sq) {
  wave_chan(m, q, c);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    slot[threadIdx.x >> 6] = m;
    slot[W + (threadIdx.x >> 6)] = q;
  }
  __syncthreads();
  float a[W], b[W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    a[i] = slot[i];
    b[i] = slot[W + i];
  }
  float cw = 64.0f * c;
#pragma unroll
  for (int h = W / 2; h >= 1; h /= 2) {
#pragma unroll
    for (int i = 0; i < h; ++i) chan_merge(a[i], b[i], a[i + h], b[i + h], 0.5f * cw);
    cw *= 2.0f;
  }
  mean = a[0];
  sq = b[0];
}

// One thread's statistics over its GPL granules: the mean, then the sum of
// squares about it.  The row stays packed between the passes and after them
// (an empty asm keeps the compiler from holding its widened floats).
template <typename T, int GPL>
__device__ __forceinline__ void thread_chan(u32x4 (&raw)[GPL], float& m, float& q) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += v[k];
  }
  // divided by the thread's element count: exactly when it is a power of two,
  // else correctly rounded (whole rows of 64 * {3, 5, 6, 7} granules)
  m = tree8(acc) / (float)(8 * GPL);
#pragma unroll
  for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(raw[g]));
  float acc2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float d = v[k] - m;
      acc2[k] = fmaf(d, d, acc2[k]);
    }
  }
  q = tree8(acc2);
#pragma unroll
  for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(raw[g]));  // and again for the output
}

// RMSNorm: the next row's loads are issued as soon as the current row's sum of
// squares is known, before its stores.  w (or ones when absent: x * 1 is
// exact, so the result equals the unweighted one) stays in registers.
template <typename T, int W, int S, bool HAS_W>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(4))) void rmsnorm_rowpipe_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, uint16_t* y, int64_t rows, int64_t xs,
    int64_t ys, float n_f, float eps) {
  constexpr int GPL = kRowpipeGpl;
  __shared__ float slot[2][S * W];  // alternate per row: a wave may start the next row's sum early
  const int t = threadIdx.x;
  const u32x4 ones = (u32x4){kOnePair<T>, kOnePair<T>, kOnePair<T>, kOnePair<T>};
  u32x4 wr[GPL], cur[GPL];
  int64_t row = blockIdx.x;
  // w and the first row interleaved, with no branch between the loads
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave * W + t;
    wr[g] = HAS_W ? ld16(w + 8 * gi) : ones;
    cur[g] = ld16_stream(x + row * xs + 8 * gi);
  }
  for (int it = 0; row < rows; row += gridDim.x, ++it) {
    // keep w packed: widening it once outside the loop would double its registers
#pragma unroll
    for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(wr[g]));
    float acc[S][8] = {};
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      float v[8];
      widen8<T>(cur[g], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[g % S][k] = fmaf(v[k], v[k], acc[g % S][k]);
    }
    float part[S];
#pragma unroll
    for (int h = 0; h < S; ++h) part[h] = tree8(acc[h]);
    const float ss = block_sum_split<W, S>(part, slot[it & 1]);
    // and widen the row again below rather than keep its 64 floats live
#pragma unroll
    for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(cur[g]));
    const float rstd = 1.0f / sqrtf(ss / n_f + eps);
    const int64_t next = row + gridDim.x;
    u32x4 nxt[GPL];
    if (next < rows) {  // uniform across the workgroup
#pragma unroll
      for (int g = 0; g < GPL; ++g) nxt[g] = ld16_stream(x + next * xs + 8 * (g * kWave * W + t));
    } else {
#pragma unroll
      for (int g = 0; g < GPL; ++g) nxt[g] = (u32x4){0u, 0u, 0u, 0u};
    }
    uint16_t* yr = y + row * ys;
#pragma unroll
    for (int g = 0; g < GPL; ++g)
      st16_stream(yr + 8 * (g * kWave * W + t), rmsnorm_granule<T>(cur[g], wr[g], true, rstd));
#pragma unroll
    for (int g = 0; g < GPL; ++g) cur[g] = nxt[g];
  }
}

// LayerNorm, with gamma and beta both given, and the same statistics as the
// row-block kernel on these rows (thread_chan, block_chan), gamma in registers and
// beta in LDS (each thread reads back only the granules it wrote, so no
// barrier guards them).  The next row's granule g is loaded right after the
// current row's granule g is stored: with all of them issued before the
// stores (as RMSNorm does) the kernel needs more than 128 VGPRs and spills,
// and on MI355X 1024 x 32768 bf16 took 27.3 us against 25.2 us this way.
template <typename T, int W>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(4))) void layernorm_rowpipe_kernel(
    const uint16_t* x, const uint16_t* __restrict__ gam, const uint16_t* __restrict__ bet,
    uint16_t* y, int64_t rows, int64_t xs, int64_t ys, float n_f, float eps) {
  constexpr int GPL = kRowpipeGpl, HT = kWave * W;
  __shared__ float slot[2][2 * W];  // alternate per row, as in the RMSNorm kernel
  extern __shared__ u32x4 beta_lds[];   // GPL * HT granules
  const int t = threadIdx.x;
  u32x4 gr[GPL], cur[GPL];
  int64_t row = blockIdx.x;
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * HT + t;
    gr[g] = ld16(gam + 8 * gi);
    beta_lds[gi] = ld16(bet + 8 * gi);
    cur[g] = ld16_stream(x + row * xs + 8 * gi);
  }
  for (int it = 0; row < rows; row += gridDim.x, ++it) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(gr[g]));
    float m, q, mean, sq;
    thread_chan<T, GPL>(cur, m, q);
    block_chan<W>(m, q, 8.0f * GPL, slot[it & 1], mean, sq);
    const float rstd = 1.0f / sqrtf(sq / n_f + eps);
#pragma unroll
    for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(cur[g]));
    const int64_t next = row + gridDim.x;
    const bool more = next < rows;  // uniform across the workgroup
    const uint16_t* xn = x + (more ? next : row) * xs;
    uint16_t* yr = y + row * ys;
    u32x4 nxt[GPL];
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * HT + t;
      st16_stream(yr + 8 * gi,
                  layernorm_out<T>(cur[g], gr[g], beta_lds[gi], true, true, mean, 0.0f, rstd));
      nxt[g] = more ? ld16_stream(xn + 8 * gi) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int g = 0; g < GPL; ++g) cur[g] = nxt[g];
  }
}

// Workgroups of one kernel resident on the current device at once (the
// runtime's occupancy figure times the CU count), cached per device; 0 if a
// query fails, which is not cached, and the row-block kernel then takes the
// call.  Raises the kernel's dynamic LDS limit to lds bytes first.
constexpr int kMaxDevices = 64;

// Compute units of the current device, cached per device; 0 if the query
// fails (not cached).
inline int device_cus() {
  static int cache[kMaxDevices];  // 0 = not known yet; benign race: every writer stores the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 0;
  }
  int* slot = dev < kMaxDevices ? &cache[dev] : nullptr;
  if (slot) {
    const int v = __atomic_load_n(slot, __ATOMIC_RELAXED);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();  // leave no error for the caller's launch check
    return 0;
  }
  if (slot) __atomic_store_n(slot, cus, __ATOMIC_RELAXED);
  return cus;
}

template <auto K>
int64_t resident_workgroups(int threads, size_t lds) {
  static int64_t cache[kMaxDevices];  // 0 = not known yet; benign race: every writer stores the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 0;
  }
  int64_t* slot = dev < kMaxDevices ? &cache[dev] : nullptr;
  if (slot) {
    const int64_t v = __atomic_load_n(slot, __ATOMIC_RELAXED);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if ((lds > 0 && hipFuncSetAttribute(reinterpret_cast<const void*>(K),
                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)lds) != hipSuccess) ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, threads, lds) != hipSuccess ||
      per_cu < 1 ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();  // leave no error for the caller's launch check
    return 0;
  }
  const int64_t v = (int64_t)per_cu * cus;
  if (slot) __atomic_store_n(slot, v, __ATOMIC_RELAXED);
  return v;
}

// Pipelining needs rows to walk: at least half the workgroups take two.
inline bool rowpipe_window(int64_t rows, int64_t cap) {
  return cap > 0 && 2 * rows >= 3 * cap && rows <= kRowpipeMaxRowsPerBlock * cap;
}

// The pipelined kernels' shape for n elements: W waves holding S row-block
// threads each, or false if n is not 8 granules per thread of the row-block
// kernel's threads (or of a pair of them).
inline bool rowpipe_shape(int64_t n, int max_waves_at_4, int* W, int* S) {
  if (n % (8 * kRowpipeGpl * kWave) != 0) return false;
  const int ng = (int)(n / 8);
  const BlockShape b = block_shape(ng, max_waves_at_4);
  if (b.waves * kWave * b.gpt != ng || kRowpipeGpl % b.gpt != 0) return false;
  *S = kRowpipeGpl / b.gpt;
  *W = b.waves / *S;
  return *W * *S == b.waves;
}

// Waves of 8 granules per thread that hold a row of n elements exactly, if
// that is 4, 8 or 16; else 0.
inline int whole_waves(int64_t n) {
  const int64_t unit = 8 * kRowpipeGpl * kWave;  // elements per wave
  const int64_t w = n % unit == 0 ? n / unit : 0;
  return w == 4 || w == 8 || w == 16 ? (int)w : 0;
}

template <typename T, int W, int S, bool HAS_W>
bool rmsnorm_rowpipe_go(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows,
                        int64_t xs, int64_t ys, float n_f, float eps, hipStream_t st) {
  constexpr auto K = rmsnorm_rowpipe_kernel<T, W, S, HAS_W>;
  const int64_t cap = resident_workgroups<K>(kWave * W, 0);
  if (!rowpipe_window(rows, cap)) return false;
  K<<<dim3((unsigned)std::min(rows, cap)), kWave * W, 0, st>>>(x, w, y, rows, xs, ys, n_f, eps);
  return true;
}

// Launch the pipelined RMSNorm kernel if it takes this shape and row count;
// false leaves the call to the row-block kernel.
template <typename T>
bool try_rmsnorm_rowpipe(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows,
                         int64_t n, int64_t xs, int64_t ys, float n_f, float eps,
                         hipStream_t st) {
  int W = 0, S = 0;
  if (!rowpipe_shape(n, kRmsMaxWavesAt4, &W, &S)) return false;
#define QRW_RMS_PIPE(WV, SV)                                                              \
  if (W == WV && S == SV)                                                                 \
    return w ? rmsnorm_rowpipe_go<T, WV, SV, true>(x, w, y, rows, xs, ys, n_f, eps, st)   \
             : rmsnorm_rowpipe_go<T, WV, SV, false>(x, w, y, rows, xs, ys, n_f, eps, st);
  QRW_RMS_PIPE(4, 2)
  QRW_RMS_PIPE(8, 2)
  QRW_RMS_PIPE(16, 1)
#undef QRW_RMS_PIPE
  return false;
}

template <typename T, int W>
bool layernorm_rowpipe_go(const uint16_t* x, const uint16_t* g, const uint16_t* b, uint16_t* y,
                          int64_t rows, int64_t xs, int64_t ys, float n_f, float eps,
                          hipStream_t st) {
  constexpr auto K = layernorm_rowpipe_kernel<T, W>;
  constexpr size_t lds = sizeof(u32x4) * kRowpipeGpl * kWave * W;
  const int64_t cap = resident_workgroups<K>(kWave * W, lds);
  if (!rowpipe_window(rows, cap)) return false;
  K<<<dim3((unsigned)std::min(rows, cap)), kWave * W, lds, st>>>(x, g, b, y, rows, xs, ys, n_f,
                                                                 eps);
  return true;
}

// The same for LayerNorm with both gamma and beta, whose row-block kernel on
// these rows has the pipelined kernel's shape.
template <typename T>
bool try_layernorm_rowpipe(const uint16_t* x, const uint16_t* g, const uint16_t* b, uint16_t* y,
                           int64_t rows, int64_t n, int64_t xs, int64_t ys, float n_f, float eps,
                           hipStream_t st) {
  if (!g || !b) return false;
  switch (whole_waves(n)) {
    case 4: return layernorm_rowpipe_go<T, 4>(x, g, b, y, rows, xs, ys, n_f, eps, st);
    case 8: return layernorm_rowpipe_go<T, 8>(x, g, b, y, rows, xs, ys, n_f, eps, st);
    case 16: return layernorm_rowpipe_go<T, 16>(x, g, b, y, rows, xs, ys, n_f, eps, st);
    default: return false;
  }
}

template <typename T, int W, int GPL, bool TAIL>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(GPL <= 4 ? (TAIL ? 7 : 8) : 4))) void layernorm_rowblock_kernel(
    const uint16_t* x, const uint16_t* __restrict__ gam, const uint16_t* __restrict__ bet,
    uint16_t* y, int nfull, int n, int64_t xs, int64_t ys, float n_f, float eps) {
  __shared__ float slot0[W], slot1[W], slot2[W];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  const bool mine = TAIL && t == nfull % (kWave * W);
  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave * W + t;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (gi < nfull) raw[g] = ld16_stream(xr + 8 * gi);
  }
  const u32x4 xt = ld_tail<TAIL>(xr, mine, nfull, n);
  // the same two-part mean as the one-wave kernel
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL + (TAIL ? 1 : 0); ++g) {
    float v[8];
    widen8<T>(g < GPL ? raw[g] : xt, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += v[k];
  }
  const float mu0 = block_sum<W>(tree8(acc), slot0) / n_f;
  float acc1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float acc2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave * W + t;
    if (gi < nfull) {
      float v[8];
      widen8<T>(raw[g], v);
      centred_moments(v, 8, mu0, acc1, acc2);
    }
  }
  if (mine) {
    float v[8];
    widen8<T>(xt, v);
    centred_moments(v, n & 7, mu0, acc1, acc2);
  }
  const float r = block_sum<W>(tree8(acc1), slot1) / n_f;
  const float m2 = block_sum<W>(tree8(acc2), slot2) / n_f;
  const float var = fmaxf(fmaf(-r, r, m2), 0.0f);
  const float rstd = 1.0f / sqrtf(var + eps);
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  if (gam && bet) {  // as in the one-wave kernel
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      if (gi < nfull)
        st16_stream(yr + 8 * gi, layernorm_out<T>(raw[g], ld16(gam + 8 * gi),
                                                  ld16(bet + 8 * gi), true, true, mu0, r, rstd));
    }
  } else {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      if (gi < nfull)
        st16_stream(yr + 8 * gi, layernorm_out<T>(raw[g], gam ? ld16(gam + 8 * gi) : zero,
                                                  bet ? ld16(bet + 8 * gi) : zero, gam != nullptr,
                                                  bet != nullptr, mu0, r, rstd));
    }
  }
  if (mine)
    st_partial(yr + 8 * nfull,
               layernorm_out<T>(xt, ld_tail<TAIL>(gam, gam != nullptr, nfull, n),
                                ld_tail<TAIL>(bet, bet != nullptr, nfull, n), gam != nullptr,
                                bet != nullptr, mu0, r, rstd),
               n & 7);
}

// The row-block kernel on rows of 8 whole granules per thread of W = 4, 8 or
// 16 waves (n = 16384, 32768, 65536): Chan statistics through one barrier,
// which the pipelined kernel reproduces bit for bit.  Measured on MI355X
// (bf16, against the two-part kernel above, which these rows took before):
// with 8 waves at 4 granules, 16384-element rows ran 0.75x as fast at 1024
// rows (1.05x at 8192); at 8 granules and up to 6 waves per SIMD, 1.00-1.04x
// from 256 to 1024 rows and 0.98x at 8192.  At 8 and 16 waves, more than 4
// waves per SIMD made it slower (640 x 32768: 0.89x; 4096 x 32768: 0.92x),
// 4 gives 1.04x and 0.98x.
template <typename T, int W, int GPL, bool EARLY>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(4, W <= 4 ? 8 : 4))) void layernorm_rowblock_chan_kernel(
    const uint16_t* x, const uint16_t* __restrict__ gam, const uint16_t* __restrict__ bet,
    uint16_t* y, int64_t xs, int64_t ys, float n_f, float eps) {
  __shared__ float slot[2 * W];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  u32x4 raw[GPL], gg[GPL], bb[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) raw[g] = ld16_stream(xr + 8 * (g * kWave * W + t));
  float m, q, mean, sq;
  thread_chan<T, GPL>(raw, m, q);
  if (EARLY) {  // gamma and beta both given
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      gg[g] = ld16(gam + 8 * (g * kWave * W + t));
      bb[g] = ld16(bet + 8 * (g * kWave * W + t));
    }
  }
  block_chan<W>(m, q, 8.0f * GPL, slot, mean, sq);
  const float rstd = 1.0f / sqrtf(sq / n_f + eps);
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  if (EARLY) {
#pragma unroll
    for (int g = 0; g < GPL; ++g)
      st16_stream(yr + 8 * (g * kWave * W + t),
                  layernorm_out<T>(raw[g], gg[g], bb[g], true, true, mean, 0.0f, rstd));
  } else if (gam && bet) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      st16_stream(yr + 8 * gi, layernorm_out<T>(raw[g], ld16(gam + 8 * gi), ld16(bet + 8 * gi),
                                                true, true, mean, 0.0f, rstd));
    }
  } else {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const int gi = g * kWave * W + t;
      st16_stream(yr + 8 * gi, layernorm_out<T>(raw[g], gam ? ld16(gam + 8 * gi) : zero,
                                                bet ? ld16(bet + 8 * gi) : zero, gam != nullptr,
                                                bet != nullptr, mean, 0.0f, rstd));
    }
  }
}

// One wave per row with Chan statistics (wave_chan, no barrier), for bf16
// rows of 512 * GPL elements, GPL <= 8, with gamma and beta both given.
// Measured on MI355X against the one-wave kernel above, which other rows keep
// (1 GiB of rotating buffers): 4096 x 4096 bf16 11.5 against 12.2 us, 16384 x
// 512 1.13x, 8192 x 1024 and 4096 x 2048 1.04x, 4096 x 8192 (16 granules)
// 0.99x; in f16 the same kernel ran 0.87-1.07x, so f16 rows keep the
// two-part mean.
// EARLY: gamma and beta are requested before the wave's reduction instead of
// at output time (120 VGPRs instead of 67: 4 waves per SIMD instead of 7).
// Both forms compute the same bits; EARLY is taken while the launch has at
// most 8 waves per CU (2 workgroups), where a wave's latency is what shows:
// rows of 4096 took 3.0 against 3.7 us at 1 row, 4.3 against 5.2 at 512, 6.5
// against 7.1 at 2048, but 10.6 against 9.1 at 3072 and 14.6 against 11.5 at
// 4096.
template <typename T, int GPL, bool EARLY>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void layernorm_chan1_kernel(
    const uint16_t* x, const uint16_t* __restrict__ gam, const uint16_t* __restrict__ bet,
    uint16_t* y, int64_t rows, int64_t xs, int64_t ys, float n_f, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  u32x4 raw[GPL], gg[GPL], bb[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) raw[g] = ld16_stream(xr + 8 * (g * kWave + lane));
  float m, q;
  thread_chan<T, GPL>(raw, m, q);
  if (EARLY) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      gg[g] = ld16(gam + 8 * (g * kWave + lane));
      bb[g] = ld16(bet + 8 * (g * kWave + lane));
    }
  }
  wave_chan(m, q, 8.0f * GPL);
  const float rstd = 1.0f / sqrtf(q / n_f + eps);
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    st16_stream(yr + 8 * gi,
                layernorm_out<T>(raw[g], EARLY ? gg[g] : ld16(gam + 8 * gi),
                                 EARLY ? bb[g] : ld16(bet + 8 * gi), true, true, m, 0.0f, rstd));
  }
}

// Launch it for rows of n = 16384, 32768 or 65536 elements (W = n / 4096
// waves; whole_waves gives W, or 0 for any other n); false otherwise.
template <typename T>
bool layernorm_rowblock_chan(int W, const uint16_t* x, const uint16_t* g, const uint16_t* bt,
                             uint16_t* y, int64_t rows, int64_t xs, int64_t ys, float n_f,
                             float eps, hipStream_t st) {
  const dim3 grid((unsigned)rows);
  const int cus = device_cus();
  // gamma and beta requested before the reduction while the launch has at most
  // 8 waves per CU (the one-wave kernel's rule): 16384-wide rows 1.03-1.11x
  // as fast up to 512 rows, 32768-wide 1.03x up to 256; at 512 x 32768
  // (16 waves per CU) 0.72x, every workgroup requesting all of gamma and
  // beta at once
  const bool early = g && bt && cus > 0 && rows * W <= 8 * (int64_t)cus;
#define QRW_LN_RB(WV)                                                                            \
  if (early) layernorm_rowblock_chan_kernel<T, WV, 8, true><<<grid, kWave * WV, 0, st>>>(x, g, bt, y, xs, ys, n_f, eps); \
  else layernorm_rowblock_chan_kernel<T, WV, 8, false><<<grid, kWave * WV, 0, st>>>(x, g, bt, y, xs, ys, n_f, eps);
  if (W == 4) { QRW_LN_RB(4) }
  else if (W == 8) { QRW_LN_RB(8) }
  else if (W == 16)  // gamma and beta at output time only: early they spill at 16 waves
    layernorm_rowblock_chan_kernel<T, 16, 8, false><<<grid, kWave * 16, 0, st>>>(x, g, bt, y, xs, ys, n_f, eps);
  else return false;
#undef QRW_LN_RB
  return true;
}

// ------------------------------------------------- split-K, two passes
// Rows beyond what a workgroup's registers hold (s3.2.4): the first pass only
// accumulates the sum of squares, chunk by chunk; the second pass walks the
// chunks in reverse order, so the chunks read last in the first pass are the
// first re-read (still in cache), and writes y.  x is read twice; the ledger
// counts that.  One 1024-thread workgroup per row; a chunk is one granule per
// thread, and the first pass keeps kSplitUnroll chunks of loads in flight.
constexpr int kSplitWaves = 16;
constexpr int kSplitThreads = kWave * kSplitWaves;
constexpr int kSplitUnroll = 4;

template <typename T, bool TAIL>
__global__ __launch_bounds__(kSplitThreads) void rmsnorm_splitk_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, uint16_t* y, int nfull, int n, int64_t xs,
    int64_t ys, float n_f, float eps) {
  __shared__ float slot[kSplitWaves];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * xs;
  uint16_t* yr = y + row * ys;
  const bool mine = TAIL && t == nfull % kSplitThreads;
  const int chunks = (nfull + kSplitThreads - 1) / kSplitThreads;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < chunks; c0 += kSplitUnroll) {
    u32x4 raw[kSplitUnroll];
#pragma unroll
    for (int u = 0; u < kSplitUnroll; ++u) {
      const int gi = (c0 + u) * kSplitThreads + t;
      raw[u] = (u32x4){0u, 0u, 0u, 0u};
      if (gi < nfull) raw[u] = ld16(xr + 8 * gi);
    }
#pragma unroll
    for (int u = 0; u < kSplitUnroll; ++u) {
      float v[8];
      widen8<T>(raw[u], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(v[k], v[k], acc[k]);
    }
  }
  if (TAIL) {  // the partial granule ends its thread's sequence
    float v[8];
    widen8<T>(ld_tail<TAIL>(xr, mine, nfull, n), v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(v[k], v[k], acc[k]);
  }
  const float ss = block_sum<kSplitWaves>(tree8(acc), slot);
  const float rstd = 1.0f / sqrtf(ss / n_f + eps);
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  if (mine)  // the last granule of the row comes first in the reversed pass
    st_partial(yr + 8 * nfull,
               rmsnorm_granule<T>(ld_partial(xr + 8 * nfull, n & 7),
                                  w ? ld_partial(w + 8 * nfull, n & 7) : zero, w != nullptr,
                                  rstd),
               n & 7);
  for (int c = chunks - 1; c >= 0; --c) {  // reverse order: the last chunks are still cached
    const int gi = c * kSplitThreads + t;
    if (gi < nfull)
      st16_stream(yr + 8 * gi, rmsnorm_granule<T>(ld16(xr + 8 * gi),
                                                  w ? ld16(w + 8 * gi) : zero, w != nullptr,
                                                  rstd));
  }
}

// ------------------------------------------------------------------ launch
namespace {

int granules_per_lane(int ng) {
  return ng <= 64 ? 1 : ng <= 128 ? 2 : ng <= 256 ? 4 : ng <= 512 ? 8 : 16;
}

// Whole rows (no partial granule) of 64 * {3, 5, 6, 7, 10, 12, 14} granules --
// hidden sizes such as 1536, 2560, 3072, 3584, 5120, 6144 and 7168 -- have
// one-wave instances of their own (full rows: no masked loads or stores, no
// idle register slots); other rows round up to 1, 2, 4, 8 or 16 granules per
// lane.  Measured on MI355X (bf16 and f16, 1024 and 4096 rows, against the
// rounded-up instance): LayerNorm 0.99-1.29x, unweighted RMSNorm 1.00-1.13x,
// RMSNorm with the weight read beside x 1.13-1.20x; RMSNorm with the weight
// read at output time (4 or more workgroups per CU) 0.88-1.16x, so that form
// keeps the rounded-up instance.  The sums are the same (the extra slots
// add zeros), so the two RMSNorm forms give the same bits.
int exact_granules(int ng, bool tail) {
  if (!tail && ng % kWave == 0) {
    const int e = ng / kWave;
    if (e == 3 || e == 5 || e == 6 || e == 7 || e == 10 || e == 12 || e == 14) return e;
  }
  return granules_per_lane(ng);
}

}  // namespace

#define QRW_NORM_DISPATCH(KERNEL, T, gpl, full, tail, grid, stream, ...)                      \
  do {                                                                                        \
    switch (gpl) {                                                                            \
      case 1:                                                                                 \
        if (tail) KERNEL<T, 1, false, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);        \
        else if (full) KERNEL<T, 1, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);   \
        else KERNEL<T, 1, false, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);           \
        break;                                                                                \
      case 2:                                                                                 \
        if (tail) KERNEL<T, 2, false, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);        \
        else if (full) KERNEL<T, 2, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);   \
        else KERNEL<T, 2, false, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);           \
        break;                                                                                \
      case 4:                                                                                 \
        if (tail) KERNEL<T, 4, false, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);        \
        else if (full) KERNEL<T, 4, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);   \
        else KERNEL<T, 4, false, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);           \
        break;                                                                                \
      /* exact_granules: whole rows only */                                                  \
      case 3: KERNEL<T, 3, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;     \
      case 5: KERNEL<T, 5, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;     \
      case 6: KERNEL<T, 6, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;     \
      case 7: KERNEL<T, 7, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;     \
      case 10: KERNEL<T, 10, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;   \
      case 12: KERNEL<T, 12, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;   \
      case 14: KERNEL<T, 14, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__); break;   \
      case 8:                                                                                 \
        if (tail) KERNEL<T, 8, false, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);        \
        else if (full) KERNEL<T, 8, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);   \
        else KERNEL<T, 8, false, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);           \
        break;                                                                                \
      default:                                                                                \
        if (tail) KERNEL<T, 16, false, true><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);       \
        else if (full) KERNEL<T, 16, true, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);  \
        else KERNEL<T, 16, false, false><<<grid, kBlock, 0, stream>>>(__VA_ARGS__);          \
        break;                                                                                \
    }                                                                                         \
  } while (0)

// One launch of a row-block kernel: W waves per workgroup, one row per workgroup.
#define QRW_ROWBLOCK_GO(KERNEL, T, W, GPL, tail, rows, stream, ...)                           \
  do {                                                                                        \
    if (tail) KERNEL<T, W, GPL, true><<<dim3((unsigned)(rows)), kWave * W, 0, stream>>>(__VA_ARGS__); \
    else KERNEL<T, W, GPL, false><<<dim3((unsigned)(rows)), kWave * W, 0, stream>>>(__VA_ARGS__);     \
  } while (0)

#define QRW_ROWBLOCK_DISPATCH(KERNEL, T, waves, gpt, tail, rows, stream, ...)                 \
  do {                                                                                        \
    if (gpt == 4) {                                                                           \
      if (waves <= 8) QRW_ROWBLOCK_GO(KERNEL, T, 8, 4, tail, rows, stream, __VA_ARGS__);      \
      else QRW_ROWBLOCK_GO(KERNEL, T, 16, 4, tail, rows, stream, __VA_ARGS__);                \
      break;                                                                                  \
    }                                                                                         \
    switch (waves) {                                                                          \
      case 2: QRW_ROWBLOCK_GO(KERNEL, T, 2, 8, tail, rows, stream, __VA_ARGS__); break;       \
      case 4: QRW_ROWBLOCK_GO(KERNEL, T, 4, 8, tail, rows, stream, __VA_ARGS__); break;       \
      case 8: QRW_ROWBLOCK_GO(KERNEL, T, 8, 8, tail, rows, stream, __VA_ARGS__); break;       \
      default: QRW_ROWBLOCK_GO(KERNEL, T, 16, 8, tail, rows, stream, __VA_ARGS__); break;     \
    }                                                                                         \
  } while (0)

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int64_t n,
                          int64_t xs, int64_t ys, int dtype, float eps, hipStream_t stream) {
  const int ng = (int)((n + 7) / 8);
  const bool tail = n % 8 != 0;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  auto* yp = static_cast<uint16_t*>(y);
  const int ni = (int)n;
  const int nfull = (int)(n >> 3);  // whole granules; the kernels take the partial one apart
  const float nf = (float)n;
  if (ng <= kOneWaveGranules) {
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    // w at output time once the launch holds 4 or more workgroups per CU
    const int cus = device_cus();
    const bool late = cus > 0 && (int64_t)grid.x >= 4 * (int64_t)cus;
    const int gpl = wp && late ? granules_per_lane(ng) : exact_granules(ng, tail);
    const bool full = !tail && ng == gpl * kWave;
    if (dtype == 1) {
      if (!wp) QRW_NORM_DISPATCH(rmsnorm_now_kernel, F16, gpl, full, tail, grid, stream, xp, wp, yp,
                                 rows, nfull, ni, xs, ys, nf, eps);
      else if (late) QRW_NORM_DISPATCH(rmsnorm_wlate_kernel, F16, gpl, full, tail, grid, stream, xp,
                                       wp, yp, rows, nfull, ni, xs, ys, nf, eps);
      else QRW_NORM_DISPATCH(rmsnorm_w_kernel, F16, gpl, full, tail, grid, stream, xp, wp, yp,
                             rows, nfull, ni, xs, ys, nf, eps);
    } else {
      if (!wp) QRW_NORM_DISPATCH(rmsnorm_now_kernel, BF16, gpl, full, tail, grid, stream, xp, wp, yp,
                                 rows, nfull, ni, xs, ys, nf, eps);
      else if (late) QRW_NORM_DISPATCH(rmsnorm_wlate_kernel, BF16, gpl, full, tail, grid, stream, xp,
                                       wp, yp, rows, nfull, ni, xs, ys, nf, eps);
      else QRW_NORM_DISPATCH(rmsnorm_w_kernel, BF16, gpl, full, tail, grid, stream, xp, wp, yp,
                             rows, nfull, ni, xs, ys, nf, eps);
    }
  } else if (ng <= kResidentGranules) {
    const bool piped =
        dtype == 1 ? try_rmsnorm_rowpipe<F16>(xp, wp, yp, rows, n, xs, ys, nf, eps, stream)
                   : try_rmsnorm_rowpipe<BF16>(xp, wp, yp, rows, n, xs, ys, nf, eps, stream);
    if (piped) return hipGetLastError();
    const BlockShape b = block_shape(ng, kRmsMaxWavesAt4);
    const int cus = device_cus();
    // bf16 only (f16 measured 0.80-0.96x with it, bf16 1.05-1.31x from 12288
    // to 32768 elements and 1 to 256 rows), and not at 16 waves x 8
    // granules, where w in registers would spill
    const bool early = dtype != 1 && wp && cus > 0 && rows * b.waves <= 8 * (int64_t)cus &&
                       !(b.waves == 16 && b.gpt == 8);
    if (dtype == 1) {
      QRW_ROWBLOCK_DISPATCH(rmsnorm_rowblock_late, F16, b.waves, b.gpt, tail, rows, stream, xp, wp, yp,
                            nfull, ni, xs, ys, nf, eps);
    } else {
      if (early)
        QRW_ROWBLOCK_DISPATCH(rmsnorm_rowblock_early, BF16, b.waves, b.gpt, tail, rows, stream, xp, wp, yp,
                              nfull, ni, xs, ys, nf, eps);
      else
        QRW_ROWBLOCK_DISPATCH(rmsnorm_rowblock_late, BF16, b.waves, b.gpt, tail, rows, stream, xp, wp, yp,
                              nfull, ni, xs, ys, nf, eps);
    }
  } else {
    const dim3 grid((unsigned)rows);
    if (dtype == 1) {
      if (tail) rmsnorm_splitk_kernel<F16, true><<<grid, kSplitThreads, 0, stream>>>(xp, wp, yp, nfull, ni, xs, ys, nf, eps);
      else rmsnorm_splitk_kernel<F16, false><<<grid, kSplitThreads, 0, stream>>>(xp, wp, yp, nfull, ni, xs, ys, nf, eps);
    } else {
      if (tail) rmsnorm_splitk_kernel<BF16, true><<<grid, kSplitThreads, 0, stream>>>(xp, wp, yp, nfull, ni, xs, ys, nf, eps);
      else rmsnorm_splitk_kernel<BF16, false><<<grid, kSplitThreads, 0, stream>>>(xp, wp, yp, nfull, ni, xs, ys, nf, eps);
    }
  }
  return hipGetLastError();
}

hipError_t launch_layernorm(const void* x, const void* g, const void* b, void* y, int64_t rows,
                            int64_t n, int64_t xs, int64_t ys, int dtype, float eps,
                            hipStream_t stream) {
  const int ng = (int)((n + 7) / 8);
  const bool tail = n % 8 != 0;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* gp = static_cast<const uint16_t*>(g);
  const auto* bp = static_cast<const uint16_t*>(b);
  auto* yp = static_cast<uint16_t*>(y);
  const int ni = (int)n;
  const int nfull = (int)(n >> 3);  // whole granules; the kernels take the partial one apart
  const float nf = (float)n;
  if (ng <= kOneWaveGranules) {
    const int gpl = exact_granules(ng, tail);
    const bool full = !tail && ng == gpl * kWave;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    if (dtype != 1 && full && gpl <= 8 && gp && bp) {  // bf16 whole affine rows: Chan statistics
      const int cus = device_cus();
      const bool early = cus > 0 && (int64_t)grid.x * kRowsPerBlock <= 8 * (int64_t)cus;
#define QRW_LN_CHAN1(GPL)                                                                       \
  if (early) layernorm_chan1_kernel<BF16, GPL, true><<<grid, kBlock, 0, stream>>>(xp, gp, bp, yp, rows, xs, ys, nf, eps); \
  else layernorm_chan1_kernel<BF16, GPL, false><<<grid, kBlock, 0, stream>>>(xp, gp, bp, yp, rows, xs, ys, nf, eps);
      switch (gpl) {
        case 1: QRW_LN_CHAN1(1) break;
        case 2: QRW_LN_CHAN1(2) break;
        case 3: QRW_LN_CHAN1(3) break;
        case 4: QRW_LN_CHAN1(4) break;
        case 5: QRW_LN_CHAN1(5) break;
        case 6: QRW_LN_CHAN1(6) break;
        case 7: QRW_LN_CHAN1(7) break;
        default: QRW_LN_CHAN1(8) break;
      }
#undef QRW_LN_CHAN1
      return hipGetLastError();
    }
    if (dtype == 1)
      QRW_NORM_DISPATCH(layernorm_kernel, F16, gpl, full, tail, grid, stream, xp, gp, bp, yp, rows,
                        nfull, ni, xs, ys, nf, eps);
    else
      QRW_NORM_DISPATCH(layernorm_kernel, BF16, gpl, full, tail, grid, stream, xp, gp, bp, yp,
                        rows, nfull, ni, xs, ys, nf, eps);
  } else {
    const bool piped =
        dtype == 1 ? try_layernorm_rowpipe<F16>(xp, gp, bp, yp, rows, n, xs, ys, nf, eps, stream)
                   : try_layernorm_rowpipe<BF16>(xp, gp, bp, yp, rows, n, xs, ys, nf, eps, stream);
    if (piped) return hipGetLastError();
    if (const int W = whole_waves(n)) {
      const bool whole =
          dtype == 1 ? layernorm_rowblock_chan<F16>(W, xp, gp, bp, yp, rows, xs, ys, nf, eps, stream)
                     : layernorm_rowblock_chan<BF16>(W, xp, gp, bp, yp, rows, xs, ys, nf, eps, stream);
      if (whole) return hipGetLastError();
    }
    const BlockShape b = block_shape(ng, kLnMaxWavesAt4);
    if (dtype == 1)
      QRW_ROWBLOCK_DISPATCH(layernorm_rowblock_kernel, F16, b.waves, b.gpt, tail, rows, stream, xp, gp, bp, yp,
                            nfull, ni, xs, ys, nf, eps);
    else
      QRW_ROWBLOCK_DISPATCH(layernorm_rowblock_kernel, BF16, b.waves, b.gpt, tail, rows, stream, xp, gp, bp,
                            yp, nfull, ni, xs, ys, nf, eps);
  }
  return hipGetLastError();
}

}  // namespace qrw
