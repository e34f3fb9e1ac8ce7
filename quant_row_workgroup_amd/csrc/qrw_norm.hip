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

template <typename T, int GPL, bool FULL, bool TAIL>
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
  const bool any = FULL || nfull > 0;  // wave-uniform
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (any) raw[g] = FULL ? ld16(xr + 8 * gi) : ld_masked<false>(xr, gi, nfull);
  }
  const u32x4 xt = ld_tail<TAIL>(xr, mine, nfull, n);
  // The weights are loaded with x, except in the ragged form, which reads
  // them at output time (measured faster there: 12.9 against 14.4 us on
  // 4096 x 4095 bf16; the other way round costs on whole rows).
  constexpr bool kPreW = !TAIL;
  if (kPreW && w) {
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
    if (w) {
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
  if (!kPreW && w) {  // late weights: the test stays outside the loop
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
        st16_stream(yr + 8 * gi, finish(raw[g], w ? wr[g] : (u32x4){0u, 0u, 0u, 0u}));
    }
  }
  if (mine) st_partial(yr + 8 * nfull, finish(xt, ld_tail<TAIL>(w, w != nullptr, nfull, n)), n & 7);
}

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

template <typename T, int W, int GPL, bool TAIL>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(GPL <= 4 ? 8 : 4))) void rmsnorm_rowblock_kernel(
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
  if (w) {  // no test per granule, so later weight loads run ahead of the math
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

// ------------------------------------------- rows of many waves, pipelined
// RMSNorm rows of exactly 8 granules per thread of W = 4, 8 or 16 waves (n =
// 16384, 32768 or 65536 elements), where the grid is only as large as the GPU
// holds at once.  Each workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x,
// ...; it issues the loads of its next row as soon as the current row's sum of
// squares is known, before the current row's stores, so that its reads overlap
// its own writes instead of every resident row loading and then every one
// storing in lock step.  w (or ones when absent: x * 1 is exact, so the result
// equals the unweighted one) stays in registers for the whole walk, and x is
// read non-temporally.
//
// Measured on MI355X against the one-row-per-workgroup kernel above (bf16, 8
// or more rotating buffer sets of at least 1 GiB in all), by rows per resident
// workgroup: from 1.5 to 4 it was 1.00-1.17x as fast (1024 x 32768 23.8
// against 25.4 us, 768 x 32768 17.0 against 19.8, 512 x 65536 23.0 against
// 25.3), at 1 or less mostly slower (512 x 32768 0.91x, 1024 x 16384 0.83x: a
// workgroup then holds one row with fewer waves than the row-block kernel), at
// 8 0.99x; rows with masked granules (1024 x 32760, 4096 x 8200, 8192 x 12288)
// were 2-4% slower.  So it takes whole rows, from 1.5 to 4 rows per resident
// workgroup.
constexpr int kRowpipeGpl = 8;
constexpr int kRowpipeMaxRowsPerBlock = 4;

template <typename T>
constexpr uint32_t kOnePair = std::is_same<T, BF16>::value ? 0x3F803F80u : 0x3C003C00u;

template <typename T, int W, bool HAS_W>
__global__ __launch_bounds__(kWave* W) __attribute__((amdgpu_waves_per_eu(4))) void rmsnorm_rowpipe_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, uint16_t* y, int64_t rows, int64_t xs,
    int64_t ys, float n_f, float eps) {
  constexpr int GPL = kRowpipeGpl;
  __shared__ float slot[2][W];  // alternate per row: a wave may start the next row's sum early
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
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      float v[8];
      widen8<T>(cur[g], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(v[k], v[k], acc[k]);
    }
    const float ss = block_sum<W>(tree8(acc), slot[it & 1]);
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

// Workgroups of one rowpipe instance resident on the current device at once
// (the runtime's occupancy figure times the CU count), cached per device; 0 if
// either query fails, which is not cached, and the row-block kernel then
// takes the call.
constexpr int kMaxDevices = 64;
template <typename T, int W, bool HAS_W>
int64_t rowpipe_capacity() {
  static int64_t cache[kMaxDevices];  // 0 = not known yet; benign race: every writer stores the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int64_t* slot = dev < kMaxDevices ? &cache[dev] : nullptr;
  if (slot) {
    const int64_t v = __atomic_load_n(slot, __ATOMIC_RELAXED);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rmsnorm_rowpipe_kernel<T, W, HAS_W>,
                                                   kWave * W, 0) != hipSuccess || per_cu < 1 ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();  // leave no error for the caller's launch check
    return 0;
  }
  const int64_t v = (int64_t)per_cu * cus;
  if (slot) __atomic_store_n(slot, v, __ATOMIC_RELAXED);
  return v;
}

template <typename T, int W, bool HAS_W>
bool rowpipe_go(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows, int64_t xs,
                int64_t ys, float n_f, float eps, hipStream_t st) {
  const int64_t cap = rowpipe_capacity<T, W, HAS_W>();
  // pipelining needs rows to walk: at least half the workgroups take two
  if (cap == 0 || 2 * rows < 3 * cap || rows > kRowpipeMaxRowsPerBlock * cap) return false;
  rmsnorm_rowpipe_kernel<T, W, HAS_W><<<dim3((unsigned)std::min(rows, cap)), kWave * W, 0, st>>>(
      x, w, y, rows, xs, ys, n_f, eps);
  return true;
}

// Launch the pipelined kernel if it takes this shape (whole rows of
// kRowpipeGpl granules per thread, n % 8 == 0); false leaves the row to the
// row-block kernel.
template <typename T>
bool try_rowpipe(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t rows, int64_t n,
                 int64_t xs, int64_t ys, float n_f, float eps, hipStream_t st) {
  constexpr int64_t unit = 8 * kRowpipeGpl * kWave;  // elements per wave
  switch (n % 8 == 0 && n % unit == 0 ? n / unit : 0) {
    case 4: return w ? rowpipe_go<T, 4, true>(x, w, y, rows, xs, ys, n_f, eps, st)
                     : rowpipe_go<T, 4, false>(x, w, y, rows, xs, ys, n_f, eps, st);
    case 8: return w ? rowpipe_go<T, 8, true>(x, w, y, rows, xs, ys, n_f, eps, st)
                     : rowpipe_go<T, 8, false>(x, w, y, rows, xs, ys, n_f, eps, st);
    case 16: return w ? rowpipe_go<T, 16, true>(x, w, y, rows, xs, ys, n_f, eps, st)
                      : rowpipe_go<T, 16, false>(x, w, y, rows, xs, ys, n_f, eps, st);
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
BlockShape block_shape(int ng, int max_waves_at_4) {
  const int gpt = ng <= max_waves_at_4 * kWave * 4 ? 4 : 8;
  int w = 2;
  while (w < 16 && w * kWave * gpt < ng) w *= 2;
  return {w, gpt};
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
    const int gpl = granules_per_lane(ng);
    const bool full = !tail && ng == gpl * kWave;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    if (dtype == 1)
      QRW_NORM_DISPATCH(rmsnorm_kernel, F16, gpl, full, tail, grid, stream, xp, wp, yp, rows, nfull,
                        ni, xs, ys, nf, eps);
    else
      QRW_NORM_DISPATCH(rmsnorm_kernel, BF16, gpl, full, tail, grid, stream, xp, wp, yp, rows, nfull,
                        ni, xs, ys, nf, eps);
  } else if (ng <= kResidentGranules) {
    const bool piped = dtype == 1 ? try_rowpipe<F16>(xp, wp, yp, rows, n, xs, ys, nf, eps, stream)
                                  : try_rowpipe<BF16>(xp, wp, yp, rows, n, xs, ys, nf, eps, stream);
    if (piped) return hipGetLastError();
    const BlockShape b = block_shape(ng, 16);
    if (dtype == 1)
      QRW_ROWBLOCK_DISPATCH(rmsnorm_rowblock_kernel, F16, b.waves, b.gpt, tail, rows, stream, xp, wp, yp, nfull,
                            ni, xs, ys, nf, eps);
    else
      QRW_ROWBLOCK_DISPATCH(rmsnorm_rowblock_kernel, BF16, b.waves, b.gpt, tail, rows, stream, xp, wp, yp, nfull,
                            ni, xs, ys, nf, eps);
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
    const int gpl = granules_per_lane(ng);
    const bool full = !tail && ng == gpl * kWave;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    if (dtype == 1)
      QRW_NORM_DISPATCH(layernorm_kernel, F16, gpl, full, tail, grid, stream, xp, gp, bp, yp, rows,
                        nfull, ni, xs, ys, nf, eps);
    else
      QRW_NORM_DISPATCH(layernorm_kernel, BF16, gpl, full, tail, grid, stream, xp, gp, bp, yp,
                        rows, nfull, ni, xs, ys, nf, eps);
  } else {
    const BlockShape b = block_shape(ng, 8);
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
