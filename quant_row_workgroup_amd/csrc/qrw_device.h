// qrw_device.h -- device primitives shared by the row-operator kernels (gfx950).
//
// * 16-byte granules: each lane moves 8 x 16-bit elements with one
//   global_load_dwordx4 / global_store_dwordx4.
// * widening of f16/bf16 to f32 (exact) and narrowing with one
//   round-to-nearest-even step (v_cvt_pk_bf16_f32, v_cvt_f16_f32).
// * wave64 reductions: a DPP butterfly inside each 16-lane row (quad_perm
//   xor-1, xor-2, half-row mirror, row mirror), then the four row results are
//   read with v_readlane and combined in a fixed order.  Every lane of a wave
//   ends with the same bits, and the reduction tree does not depend on the
//   launch shape, so a row gives the same result in any batch.
// * E4M3FN packing with v_cvt_pk_fp8_f32 (OCP FP8 on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace qrw {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- memory
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
// Streaming forms (non-temporal hint): data touched once per launch.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ void st8_stream(void* p, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// The first `cnt` (0..7) 16-bit elements at p (16-byte aligned) as one
// granule, the rest zero, in at most three accesses of 4, 2 and 1 elements
// (the bits of cnt); nothing at or past p + cnt is read.  (A row's partial
// last granule: its padding contributes zero to every sum.)  Measured on
// MI355X: one access per element made 4096 x 4095 bf16 RMSNorm 13.2 us, this
// 12.1 us; without the partial granule at all (a timing probe) it is 11.2 us.
__device__ __forceinline__ u32x4 ld_partial(const uint16_t* p, int cnt) {
  u32x4 g = (u32x4){0u, 0u, 0u, 0u};
  const int a = cnt & 4, b = cnt & 2;
  if (a) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    g[0] = v[0];
    g[1] = v[1];
  }
  if (b) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p + a);
    if (a) g[2] = v;
    else g[0] = v;
  }
  if (cnt & 1) {
    const uint32_t v = p[a + b];
    switch ((a + b) >> 1) {
      case 0: g[0] = v; break;
      case 1: g[1] = v; break;
      case 2: g[2] = v; break;
      default: g[3] = v; break;
    }
  }
  return g;
}
// Store the first `cnt` (0..7) elements of a granule the same way; nothing
// at or past p + cnt is written.
__device__ __forceinline__ void st_partial(uint16_t* p, u32x4 g, int cnt) {
  const int a = cnt & 4, b = cnt & 2;
  if (a) *reinterpret_cast<u32x2*>(p) = (u32x2){g[0], g[1]};
  if (b) *reinterpret_cast<uint32_t*>(p + a) = a ? g[2] : g[0];
  if (cnt & 1) {
    const int k = (a + b) >> 1;
    const uint32_t v = k == 0 ? g[0] : k == 1 ? g[1] : k == 2 ? g[2] : g[3];
    p[a + b] = (uint16_t)(v & 0xFFFFu);
  }
}

// ------------------------------------------------------- element formats
struct F16 {
  static __device__ __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
    return __builtin_bit_cast(uint32_t, h);
  }
};

struct BF16 {
  static __device__ __forceinline__ float lo(uint32_t u) {
    return __builtin_bit_cast(float, u << 16);
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return __builtin_bit_cast(float, u & 0xFFFF0000u);
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
  }
};

// Widen one granule (8 elements) to f32.
template <typename T>
__device__ __forceinline__ void widen8(u32x4 g, float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = T::lo(g[k]);
    v[2 * k + 1] = T::hi(g[k]);
  }
}

// Narrow 8 f32 values to one granule.
template <typename T>
__device__ __forceinline__ u32x4 narrow8(const float (&v)[8]) {
  u32x4 g;
#pragma unroll
  for (int k = 0; k < 4; ++k) g[k] = T::pack(v[2 * k], v[2 * k + 1]);
  return g;
}

// Eight f32 table entries starting at element 8*s of a table row.  (The
// entries are read as float vectors: __builtin_bit_cast applied directly to an
// element of an ext_vector_type value reads the wrong lane with this compiler,
// so no vector element is ever bit-cast in place.)
template <typename CS>
struct Table8;
template <>
struct Table8<float> {
  static __device__ __forceinline__ void load(const void* row, int s, float (&v)[8]) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row) + 2 * s;
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
  }
};
// Four table entries starting at element 4*j of a table row.
template <typename CS>
struct Table4;
template <>
struct Table4<float> {
  static __device__ __forceinline__ void load(const void* row, int j, float (&v)[4]) {
    const f32x4 a = reinterpret_cast<const f32x4*>(row)[j];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = a[k];
  }
};
template <typename T>
struct Table4 {
  static __device__ __forceinline__ void load(const void* row, int j, float (&v)[4]) {
    const u32x2 a = reinterpret_cast<const u32x2*>(row)[j];
    const uint32_t a0 = a[0], a1 = a[1];
    v[0] = T::lo(a0);
    v[1] = T::hi(a0);
    v[2] = T::lo(a1);
    v[3] = T::hi(a1);
  }
};

template <>
struct Table8<F16> {
  static __device__ __forceinline__ void load(const void* row, int s, float (&v)[8]) {
    widen8<F16>(ld16(reinterpret_cast<const uint16_t*>(row) + 8 * s), v);
  }
};
template <>
struct Table8<BF16> {
  static __device__ __forceinline__ void load(const void* row, int s, float (&v)[8]) {
    widen8<BF16>(ld16(reinterpret_cast<const uint16_t*>(row) + 8 * s), v);
  }
};

// Start of token t's row of a packed [tokens, half] cos or sin table.
template <typename CS>
__device__ __forceinline__ const char* table_row(const void* base, int64_t t, int half) {
  constexpr int bytes = std::is_same<CS, float>::value ? 4 : 2;
  return static_cast<const char*>(base) + t * (int64_t)half * bytes;
}

// Round eight binary32 values to the 16-bit format T (nearest-even) and back.
template <typename T>
__device__ __forceinline__ void round8(float (&v)[8]) {
  widen8<T>(narrow8<T>(v), v);
}
// bf16: one v_cvt_pk_bf16_f32 per element.  The pair (0, v) packed to bf16
// and read back as one binary32 word is RN_bf16(v) itself (bf16 is the upper
// half of binary32; the lower half is the packed zero), so no widening step is
// needed.  NaN, infinities and signed zeros give the same words as the
// narrow-then-widen form.
template <>
__device__ __forceinline__ void round8<BF16>(float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bf16x2 h = __builtin_convertvector((f32x2){0.0f, v[k]}, bf16x2);
    v[k] = __builtin_bit_cast(float, h);
  }
}

// ----------------------------------------------------------- wave64 reductions
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16

// Value of lane (l ^ X) for lane l, for the partner distances of the NeoX
// pairing in the contiguous layout: DPP quad permutes for 1 and 2, a DPP
// rotate by 8 inside each 16-lane row for 8 (which is xor 8 there), and the
// LDS crossbar (ds_swizzle, bit mode) for 4 and 16.
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(X == 1 || X == 2 || X == 4 || X == 8 || X == 16, "unsupported distance");
  if constexpr (X == 1) return dpp<kDppXor1>(v);
  else if constexpr (X == 2) return dpp<kDppXor2>(v);
  else if constexpr (X == 8) return dpp<0x128>(v);  // row_ror:8
  else
    return __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (X << 10)));
}

// Sum over the 64 lanes; every lane receives the same value.  All lanes must
// be active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Max over the 64 lanes (inputs are >= 0 or -0).  All lanes must be active.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// Sum / max over aligned groups of L consecutive lanes (L = 1, 2, 4, ..., 64);
// every lane of a group receives the group's value.  All lanes must be active.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp<kDppXor1>(v);
  if constexpr (L >= 4) v += dpp<kDppXor2>(v);
  if constexpr (L >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp<kDppMirror>(v);
  if constexpr (L >= 32) v += lane_xor<16>(v);
  if constexpr (L >= 64) v = lane_value(v, 0) + lane_value(v, 32);
  return v;
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if constexpr (L >= 32) v = fmaxf(v, lane_xor<16>(v));
  if constexpr (L >= 64) v = fmaxf(lane_value(v, 0), lane_value(v, 32));
  return v;
}

// RN(x / s) given y = RN(1 / s), without a division (Markstein's correction:
// q = RN(x*y), the remainder q*s - x is exact by one fma, and RN(q - r*y) is
// the correctly rounded quotient for the |x| <= 448*s range of a quantiser).
// Taking the remainder with this sign keeps the sign of a zero x with no
// extra instruction: for x = -0 both fma results are -0, for x = +0 both +0.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = fmaf(q, s, -x);
  return fmaf(-r, y, q);
}

// The quantiser's scale RN(a / 448), a >= 1e-4 finite, by the same correction
// with the constant RN(1/448); equal to the correctly rounded quotient for
// every binary32 a in [2^-14, 2^128): tests/test_gpu_recip.py sweeps every
// such a on the GPU against the binary32 value nearest the binary64 quotient.
__device__ __forceinline__ float scale_e4m3(float a) {
  constexpr float kInv = 1.0f / 448.0f;  // folded correctly rounded
  return div_rn(a, 448.0f, kInv);
}

// RN(1 / s) for s in [2^-23, 2^120): the hardware reciprocal refined by one
// Newton step, y0 + y0 (1 - s y0).  On gfx950 this equals the IEEE quotient
// 1.0f / s for every binary32 s in that range, in three instructions instead
// of the division sequence: tests/test_gpu_recip.py sweeps every such s on the
// GPU (about 1.2e9 values) against the binary32 value nearest the binary64
// quotient.  A scale of a finite amax is in the range: max(amax, 1e-4) / 448
// >= 2^-22.  div_rn's correction relies on this reciprocal being correctly
// rounded.
__device__ __forceinline__ float recip_rn(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  return fmaf(fmaf(-s, y0, 1.0f), y0, y0);
}

// Sum of squares of the two 16-bit elements of a packed pair, added to acc,
// in one v_dot2c_f32_{bf16,f16}: the products of 16-bit values are exact in
// binary32.  (The pair is taken by value: see the note on Table8<float>.)
__device__ __forceinline__ float sumsq2(F16, uint32_t u, float acc) {
  const f16x2 h = __builtin_bit_cast(f16x2, u);
  return __builtin_amdgcn_fdot2(h, h, acc, false);
}
__device__ __forceinline__ float sumsq2(BF16, uint32_t u, float acc) {
  const bf16x2 h = __builtin_bit_cast(bf16x2, u);
  return __builtin_amdgcn_fdot2_f32_bf16(h, h, acc, false);
}

// Pairwise sum of eight per-slot partial sums, in a fixed tree.
__device__ __forceinline__ float tree8(const float (&a)[8]) {
  return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// ----------------------------------------------------------------- FP8
// Eight f32 values (already scaled into [-448, 448]) to eight E4M3FN codes,
// element k in byte k.
// Each conversion writes one 16-bit half of its destination and keeps the
// other; the first of each pair starts from v[0] (resp. v[4]) as the kept half,
// which the second overwrites, so no destination needs zeroing first.
__device__ __forceinline__ u32x2 fp8x8(const float (&v)[8]) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], __builtin_bit_cast(int, v[0]), false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], __builtin_bit_cast(int, v[4]), false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
  return (u32x2){(uint32_t)lo, (uint32_t)hi};
}

}  // namespace qrw
