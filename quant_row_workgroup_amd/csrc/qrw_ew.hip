// qrw_ew.hip -- elementwise y = cast(x * alpha + b) over flat arrays (gfx950).
//
// Definition: "TileLang tutorial, ch. 13", s3.1.1 (a + b; (x * alpha) cast to
// the output dtype) and s1.2's scale+add scenario (y = x * a + b), rounded once
// to the output dtype:
// * fp32 output: one binary32 fma, which is the correctly rounded result;
// * 16-bit output: one binary64 fma (exact for 16-bit operands, and for fp32
//   operands unless the addend is below 2^-5 of the product's last bit), then
//   the binary64 value is rounded to odd at binary32 precision, and that is
//   cast once, nearest-even, to the 16-bit format.  A value rounded to odd with
//   two or more extra bits rounds like the value itself (Boldo and Melquiond,
//   IEEE TC 2008), so the output is the rounding of the binary64 result rather
//   than a double rounding through binary32.  The HBM-bound kernel hides the
//   few extra binary64 operations.  A plain sum of two 16-bit values (alpha
//   == 1) skips binary64: its binary32 sum rounds correctly (see combine).
//
// Mapping: lane l of wave w takes E consecutive elements at
// ((w * U + u) * 64 + l) * E for u < U, so every memory instruction of a wave
// covers 64 * E contiguous elements.  E = 8 when every operand is 16-bit (one
// 16-byte granule per operand), E = 4 when any operand is fp32 (16 bytes of
// fp32, 8 bytes of a 16-bit type), so a mixed-width cast still moves whole
// 16-byte (or 8-byte) vectors (s3.1.5: a cross-dtype cast is limited by the
// wider side).  Only the one unit that straddles the end of the array is done
// element by element; all other units keep their vector loads and stores
// whatever n is (s5.1: a ragged length must not turn the body scalar).
// Inputs are read and outputs written with non-temporal hints.
#include <type_traits>

#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

// Scalar element access (the ragged tail).
template <typename T>
struct Scalar;
template <>
struct Scalar<float> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <typename T>
struct Scalar {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return T::lo(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)(T::pack(v, 0.0f) & 0xFFFFu);
  }
};

// E consecutive elements starting at element i: a raw vector load (kept as
// loaded until its unit is computed) and its widening, and a narrowing store.
template <typename T, int E>
struct Vec;
template <>
struct Vec<float, 4> {
  using Raw = f32x4;
  static __device__ __forceinline__ Raw ld(const void* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + i / 4);
  }
  static __device__ __forceinline__ void widen(Raw a, float (&v)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = a[k];
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, const float (&v)[4]) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p) + i / 4);
  }
};
template <typename T>
struct Vec<T, 4> {
  using Raw = u32x2;
  static __device__ __forceinline__ Raw ld(const void* p, int64_t i) {
    return ld8_stream(static_cast<const uint16_t*>(p) + i);
  }
  static __device__ __forceinline__ void widen(Raw a, float (&v)[4]) {
    const uint32_t a0 = a[0], a1 = a[1];
    v[0] = T::lo(a0);
    v[1] = T::hi(a0);
    v[2] = T::lo(a1);
    v[3] = T::hi(a1);
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, const float (&v)[4]) {
    const u32x2 a = {T::pack(v[0], v[1]), T::pack(v[2], v[3])};
    st8_stream(static_cast<uint16_t*>(p) + i, a);
  }
};
template <typename T>
struct Vec<T, 8> {
  using Raw = u32x4;
  static __device__ __forceinline__ Raw ld(const void* p, int64_t i) {
    return ld16_stream(static_cast<const uint16_t*>(p) + i);
  }
  static __device__ __forceinline__ void widen(Raw a, float (&v)[8]) { widen8<T>(a, v); }
  static __device__ __forceinline__ void st(void* p, int64_t i, const float (&v)[8]) {
    st16_stream(static_cast<uint16_t*>(p) + i, narrow8<T>(v));
  }
};

// binary64 -> binary32 rounded to odd: the truncation, with its last bit set
// when the conversion is inexact.
__device__ __forceinline__ float round_odd_f32(double d) {
  const float f = (float)d;
  if ((double)f == d) return f;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 1u) == 0) u = fabs(d) > fabs((double)f) ? u + 1 : u - 1;
  return __builtin_bit_cast(float, u);
}

// x * alpha (+ b) for an output of type YT, in the form the YT store expects.
// ADD: x + b of two values of the 16-bit output format (alpha == 1).  Their
// binary32 sum rounds once more to that format exactly as the exact sum does:
// it is exact when the exponents differ by at most 15 (bf16) or 13 (f16), and
// otherwise the smaller operand is below a quarter of the larger one's half
// ulp, so that both the exact and the binary32 sums round to the larger.
template <typename YT, bool HAS_B, bool ADD = false>
__device__ __forceinline__ float combine(float x, float alpha, float b) {
  if constexpr (ADD) {
    return x + b;
  } else if constexpr (std::is_same<YT, float>::value) {
    return HAS_B ? fmaf(x, alpha, b) : x * alpha;
  } else {
    const double v = HAS_B ? fma((double)x, (double)alpha, (double)b) : (double)x * (double)alpha;
    return round_odd_f32(v);
  }
}

template <typename XT, typename YT, bool HAS_B, int E, int U, bool ADD>
__global__ __launch_bounds__(kBlock) void ew_kernel(const void* __restrict__ x,
                                                    const void* __restrict__ b, void* y,
                                                    int64_t n, float alpha) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  using V = Vec<XT, E>;
  typename V::Raw xr[U], br[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = ((wave * U + u) * kWave + lane) * E;
    if (i + E <= n) {
      xr[u] = V::ld(x, i);
      if (HAS_B) br[u] = V::ld(b, i);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = ((wave * U + u) * kWave + lane) * E;
    if (i + E <= n) {
      float xv[E], bv[E], yv[E];
      V::widen(xr[u], xv);
      if (HAS_B) V::widen(br[u], bv);
#pragma unroll
      for (int e = 0; e < E; ++e) yv[e] = combine<YT, HAS_B, ADD>(xv[e], alpha, HAS_B ? bv[e] : 0.0f);
      Vec<YT, E>::st(y, i, yv);
    } else if (i < n) {  // the unit that straddles the end
      for (int64_t k = i; k < n; ++k) {
        const float xs = Scalar<XT>::ld(x, k);
        Scalar<YT>::st(y, k, combine<YT, HAS_B, ADD>(xs, alpha, HAS_B ? Scalar<XT>::ld(b, k) : 0.0f));
      }
    }
  }
}

// ------------------------------------------------------------------ launch
namespace {

constexpr int64_t kEwBigUnits = (int64_t)1 << 20;  // above this, 4 units per lane

template <typename XT, typename YT, bool HAS_B, int E, bool ADD = false>
void ew_go(const void* x, const void* b, void* y, int64_t n, float alpha, hipStream_t st) {
  const int64_t units = (n + E - 1) / E;
  if (units > kEwBigUnits) {
    constexpr int U = 4;
    const int64_t waves = (units + kWave * U - 1) / (kWave * U);
    const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
    ew_kernel<XT, YT, HAS_B, E, U, ADD><<<grid, kBlock, 0, st>>>(x, b, y, n, alpha);
  } else {
    const int64_t waves = (units + kWave - 1) / kWave;
    const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
    ew_kernel<XT, YT, HAS_B, E, 1, ADD><<<grid, kBlock, 0, st>>>(x, b, y, n, alpha);
  }
}

template <typename XT, typename YT>
void ew_b(bool has_b, const void* x, const void* b, void* y, int64_t n, float alpha,
          hipStream_t st) {
  constexpr bool kWide = std::is_same<XT, float>::value || std::is_same<YT, float>::value;
  constexpr int E = kWide ? 4 : 8;
  if constexpr (std::is_same<XT, YT>::value) {  // an addend only comes with one dtype
    if (has_b) {
      if (!kWide && alpha == 1.0f)  // a plain 16-bit sum: binary32 is enough
        ew_go<XT, YT, true, E, true>(x, b, y, n, alpha, st);
      else
        ew_go<XT, YT, true, E>(x, b, y, n, alpha, st);
      return;
    }
  }
  ew_go<XT, YT, false, E>(x, b, y, n, alpha, st);
}

template <typename XT>
void ew_y(int y_dtype, bool has_b, const void* x, const void* b, void* y, int64_t n, float alpha,
          hipStream_t st) {
  if (y_dtype == 1)
    ew_b<XT, F16>(has_b, x, b, y, n, alpha, st);
  else if (y_dtype == 2)
    ew_b<XT, BF16>(has_b, x, b, y, n, alpha, st);
  else
    ew_b<XT, float>(has_b, x, b, y, n, alpha, st);
}

}  // namespace

hipError_t launch_ew(const void* x, const void* b, void* y, int64_t n, float alpha, int x_dtype,
                     int y_dtype, hipStream_t stream) {
  if (x_dtype == 1)
    ew_y<F16>(y_dtype, b != nullptr, x, b, y, n, alpha, stream);
  else if (x_dtype == 2)
    ew_y<BF16>(y_dtype, b != nullptr, x, b, y, n, alpha, stream);
  else
    ew_y<float>(y_dtype, b != nullptr, x, b, y, n, alpha, stream);
  return hipGetLastError();
}

}  // namespace qrw
