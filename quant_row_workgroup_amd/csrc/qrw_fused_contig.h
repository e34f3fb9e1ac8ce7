// qrw_fused_contig.h -- the fused RMSNorm -> RoPE -> per-token E4M3 operator
// in the contiguous layout, for the shapes where every head rotates whole
// (gfx950).  The benchmark shape (4096 tokens x 32 heads x 128, NeoX) takes
// this kernel.
//
// Definition: "TileLang tutorial, ch. 13", s3.3.4 (RMSNorm, RoPE on each head,
// s3.3.1, then the per-token cast of s3.1.5).
//
// The operator when every head rotates whole (rope_dim == head_dim), a head is
// 2*XD granules with XD = head_dim/16 in {1, 2, 4, 8, 16}, and the row is G
// whole wave blocks (n == 512 * G).  Lane l takes granules l, l+64, ..., so
// every load and store instruction of the wave covers one contiguous block
// (1 KiB of x, 512 B of codes).  A head then occupies 2*XD consecutive lanes:
// in the NeoX pairing the partner of lane l is lane l ^ XD, read with a lane
// exchange (lane_xor); in the interleaved pairing both members of a pair sit
// in the same granule.  Each lane needs a single table granule per token.
// The arithmetic is that of rotate(): first of a pair x_a c - x_b s as
// fma(x_a, c, x_b * (-s)), second x_b c + x_a s as fma(x_b, c, x_a * s).
//
// The token body is a device function so that a timing probe can instantiate
// the same code with per-wave timestamps (TL = true: the constant 100 MHz
// clock at entry, once the row's sum of squares is known, after the last
// store is issued, and once the wave's stores have completed).  With TL =
// false, as in the library's kernel, the hooks compile to nothing.
#pragma once

#include "qrw_device.h"

namespace qrw {

// Rows (waves) per workgroup: 4.  Measured on 4096 x 4096 bf16 (same-box
// A/B): the exact form 11.0 us at 4 rows against 11.1-11.3 at 8 and 11.5-12.1
// at 16; the staged form 11.03 at 4 against 11.03-11.08 at 8 and 11.42 at 16
// (with the one-stride instance and non-temporal code stores).
constexpr int kContigRows = 4;

// Timeline slots per wave (TL = true).
constexpr int kTimelineSlots = 4;

__device__ __forceinline__ uint64_t realtime() { return __builtin_amdgcn_s_memrealtime(); }

// PAIR: the token's row is 2 * G blocks of 512 channels, and two waves of the
// workgroup take one half each (half = 0 or 1): they exchange the sum of
// squares and the amax through pair_slot (4 floats: [half] sums, [2 + half]
// maxima) behind one workgroup barrier each, so every wave of the workgroup
// must reach both barriers -- a wave of a token past the end passes live =
// false and touches no memory.  The sum is slot[0] + slot[1] in that order.
template <typename T, typename CS, bool NEOX, int G, bool HAS_W, int XD, bool MID, bool TL,
          bool PAIR = false>
__device__ __forceinline__ void contig_token(const uint16_t* x, const uint16_t* __restrict__ w,
                                             const void* cosv, const void* sinv, uint8_t* q,
                                             float* scales, int64_t t, int64_t xs, int64_t qs,
                                             float eps, int lane, uint64_t* stamps,
                                             int half = 0, bool live = true,
                                             float* pair_slot = nullptr) {
  uint64_t t0 = 0, t1 = 0, t2 = 0;
  if (TL) t0 = realtime();
  const int64_t c0 = PAIR ? (int64_t)half * (512 * G) : 0;  // first channel of this wave's part
  const uint16_t* xr = x + t * xs + c0;
  uint8_t* qr = q + t * qs + c0;
  if (PAIR && HAS_W) w += c0;
  const int j = lane & (2 * XD - 1);  // granule index inside the head

  u32x4 r[G], wr[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    r[g] = (u32x4){0u, 0u, 0u, 0u};
    if (!PAIR || live) r[g] = ld16_stream(xr + 8 * (kWave * g + lane));
  }
  if (HAS_W) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      wr[g] = (u32x4){0u, 0u, 0u, 0u};
      if (!PAIR || live) wr[g] = ld16(w + 8 * (kWave * g + lane));
    }
  }
  float c[8], sn[8];
  // a table row holds head_dim / 2 = 8 * XD entries (a token past the end
  // reads token 0's row, which exists: tokens >= 1 whenever a kernel runs)
  const char* crow = table_row<CS>(cosv, PAIR && !live ? 0 : t, 8 * XD);
  const char* srow = table_row<CS>(sinv, PAIR && !live ? 0 : t, 8 * XD);
  if (NEOX) {
    Table8<CS>::load(crow, j & (XD - 1), c);
    Table8<CS>::load(srow, j & (XD - 1), sn);
    if (j < XD) {  // first half of the head: y = x c - x_partner s
#pragma unroll
      for (int e = 0; e < 8; ++e) sn[e] = -sn[e];
    }
  } else {
    float c4[4], s4[4];
    Table4<CS>::load(crow, j, c4);
    Table4<CS>::load(srow, j, s4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[k] = c4[k];
      sn[k] = s4[k];
    }
  }

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[(2 * g + k) & 7] = sumsq2(T{}, r[g][k], acc[(2 * g + k) & 7]);
  }
  float ss = wave_sum(tree8(acc));
  if constexpr (PAIR) {
    if (lane == 0) pair_slot[half] = ss;
    __syncthreads();
    ss = pair_slot[0] + pair_slot[1];
  }
  if (TL) t1 = realtime();
  // the mean: ss / n, n = 512 * G (1024 * G in pairs; for a power of two an
  // exact scaling)
  const float rstd = 1.0f / sqrtf(ss / (float)((PAIR ? 1024 : 512) * G) + eps);

  float v[G][8];
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    widen8<T>(r[g], v[g]);
    if (HAS_W) {
      float f[8];
      widen8<T>(wr[g], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[g][e] *= f[e];
    }
    if (MID) {  // the staged form: store x*w*rstd in T
#pragma unroll
      for (int e = 0; e < 8; ++e) v[g][e] *= rstd;
      round8<T>(v[g]);
    }
    if (NEOX) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[g][e] = fmaf(v[g][e], c[e], lane_xor<XD>(v[g][e]) * sn[e]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = v[g][2 * k], x1 = v[g][2 * k + 1];
        v[g][2 * k] = fmaf(x0, c[k], -(x1 * sn[k]));
        v[g][2 * k + 1] = fmaf(x1, c[k], x0 * sn[k]);
      }
    }
    if (MID) round8<T>(v[g]);
    // running max of |v| in four chains, each step one v_max3_f32 with
    // absolute-value source modifiers
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      m[(e >> 1) & 3] = fmaxf(fmaxf(m[(e >> 1) & 3], fabsf(v[g][e])), fabsf(v[g][e + 1]));
  }
  const float amax = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  float amax_w = wave_max(amax);
  if constexpr (PAIR) {
    if (lane == 0) pair_slot[2 + half] = amax_w;
    __syncthreads();
    amax_w = fmaxf(pair_slot[2], pair_slot[3]);
  }
  const float amax_z = MID ? amax_w : amax_w * rstd;
  const float scale = scale_e4m3(fmaxf(amax_z, 1e-4f));
  const float kq = rstd / scale;
  const float inv = recip_rn(scale);
  if (lane == 0 && (!PAIR || (live && half == 0))) scales[t] = scale;

#pragma unroll
  for (int g = 0; g < G; ++g) {
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = MID ? div_rn(v[g][e], scale, inv) : v[g][e] * kq;
    // codes: plain stores for the exact form, non-temporal for the staged one
    // (each measured faster on 4096 x 4096 bf16: 10.97 against 11.45 us, and
    // 12.29 against 12.71 us)
    if (PAIR && !live) continue;
    if (MID)
      st8_stream(qr + 8 * (kWave * g + lane), fp8x8(a));
    else
      st8(qr + 8 * (kWave * g + lane), fp8x8(a));
  }
  if (TL) {
    t2 = realtime();
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): this wave's stores are done
    const uint64_t t3 = realtime();
    if (lane == 0) {
      uint64_t* p = stamps + t * kTimelineSlots;
      p[0] = t0;
      p[1] = t1;
      p[2] = t2;
      p[3] = t3;
    }
  }
}

// ------------------------------------------------------------------ kernel
// One wave per token, kContigRows tokens per workgroup.  PACKED: the codes'
// row stride is x's (one stride for both: a packed call, the benchmark's
// included), which measured faster than two separate strides on 4096 x 4096
// bf16 (same-box A/B: the exact form 10.37 against 10.62 us, the staged form
// 11.03 against 11.6 us), since the scheduler then issues the row's loads in a
// better order.
template <typename T, typename CS, bool NEOX, int G, bool HAS_W, int XD, bool MID, bool PACKED>
__global__ __launch_bounds__(kWave * kContigRows) void rmsnorm_rope_fp8_contig_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const void* cosv, const void* sinv,
    uint8_t* q, float* scales, int64_t tokens, int64_t xs, int64_t qs, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kContigRows + (threadIdx.x >> 6);
  if (t >= tokens) return;
  contig_token<T, CS, NEOX, G, HAS_W, XD, MID, false>(x, w, cosv, sinv, q, scales, t, xs,
                                                       PACKED ? xs : qs, eps, lane, nullptr);
}

// Rows of 2 * G blocks (G = 5, 6, 7, 8: 5120 to 8192 channels), heads of 64 or
// 128: two waves per token, kPairRows tokens per workgroup.  Two tokens (4
// waves) measured fastest of 1, 2 and 4 (MI355X, 4096 tokens bf16: 48 heads of
// 128 18.3 against 22.6 us at 4, 64 heads 20.9 against 22.1 us; every barrier
// waits for all the workgroup's waves), and capping registers at 4 waves per
// SIMD made the 6-block form spill and run slower.
constexpr int kPairRows = 2;

template <typename T, typename CS, bool NEOX, int G, bool HAS_W, int XD, bool MID, bool PACKED>
__global__ __launch_bounds__(2 * kWave * kPairRows) void rmsnorm_rope_fp8_pair_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const void* cosv, const void* sinv,
    uint8_t* q, float* scales, int64_t tokens, int64_t xs, int64_t qs, float eps) {
  __shared__ float slot[kPairRows][4];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int k = wv >> 1;  // token slot in the workgroup
  const int64_t t = (int64_t)blockIdx.x * kPairRows + k;
  // no early return: both halves of every slot reach the two barriers
  contig_token<T, CS, NEOX, G, HAS_W, XD, MID, false, true>(
      x, w, cosv, sinv, q, scales, t, xs, PACKED ? xs : qs, eps, lane, nullptr, wv & 1,
      t < tokens, slot[k]);
}

template <typename T, typename CS, bool NEOX, int G, int XD>
hipError_t pair_launch(const uint16_t* x, const uint16_t* w, const void* c, const void* s,
                       uint8_t* q, float* sc, int64_t tokens, int64_t xs, int64_t qs, float eps,
                       bool mid, hipStream_t st) {
  const dim3 grid((unsigned)((tokens + kPairRows - 1) / kPairRows));
  const dim3 block(2 * kWave * kPairRows);
#define QRW_PAIR(HW, M, P) \
  rmsnorm_rope_fp8_pair_kernel<T, CS, NEOX, G, HW, XD, M, P><<<grid, block, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, eps)
  if (mid) {
    if (w && qs == xs) QRW_PAIR(true, true, true);
    else if (w) QRW_PAIR(true, true, false);
    else QRW_PAIR(false, true, false);
  } else {
    if (w && qs == xs) QRW_PAIR(true, false, true);
    else if (w) QRW_PAIR(true, false, false);
    else QRW_PAIR(false, false, false);
  }
#undef QRW_PAIR
  return hipGetLastError();
}

template <typename T, typename CS, bool NEOX, int G>
hipError_t pair_launch_xd(const uint16_t* x, const uint16_t* w, const void* c, const void* s,
                          uint8_t* q, float* sc, int64_t tokens, int64_t head_dim, int64_t xs,
                          int64_t qs, float eps, bool mid, hipStream_t st) {
  if (head_dim == 64) return pair_launch<T, CS, NEOX, G, 4>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
  return pair_launch<T, CS, NEOX, G, 8>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
}

template <typename T, typename CS, bool NEOX, int G, int XD>
hipError_t contig_launch(const uint16_t* x, const uint16_t* w, const void* c, const void* s,
                         uint8_t* q, float* sc, int64_t tokens, int64_t xs, int64_t qs, float eps,
                         bool mid, hipStream_t st) {
  const dim3 grid((unsigned)((tokens + kContigRows - 1) / kContigRows));
  const dim3 block(kWave * kContigRows);
  // the packed instances are the weighted ones (the usual call); the rest take
  // two strides
  if (mid) {
    if (w && qs == xs)
      rmsnorm_rope_fp8_contig_kernel<T, CS, NEOX, G, true, XD, true, true><<<grid, block, 0, st>>>(
          x, w, c, s, q, sc, tokens, xs, qs, eps);
    else if (w)
      rmsnorm_rope_fp8_contig_kernel<T, CS, NEOX, G, true, XD, true, false><<<grid, block, 0, st>>>(
          x, w, c, s, q, sc, tokens, xs, qs, eps);
    else
      rmsnorm_rope_fp8_contig_kernel<T, CS, NEOX, G, false, XD, true, false><<<grid, block, 0, st>>>(
          x, w, c, s, q, sc, tokens, xs, qs, eps);
  } else {
    if (w && qs == xs)
      rmsnorm_rope_fp8_contig_kernel<T, CS, NEOX, G, true, XD, false, true><<<grid, block, 0, st>>>(
          x, w, c, s, q, sc, tokens, xs, qs, eps);
    else if (w)
      rmsnorm_rope_fp8_contig_kernel<T, CS, NEOX, G, true, XD, false, false><<<grid, block, 0, st>>>(
          x, w, c, s, q, sc, tokens, xs, qs, eps);
    else
      rmsnorm_rope_fp8_contig_kernel<T, CS, NEOX, G, false, XD, false, false><<<grid, block, 0, st>>>(
          x, w, c, s, q, sc, tokens, xs, qs, eps);
  }
  return hipGetLastError();
}

template <typename T, typename CS, bool NEOX, int G>
hipError_t contig_launch_xd(const uint16_t* x, const uint16_t* w, const void* c, const void* s,
                            uint8_t* q, float* sc, int64_t tokens, int64_t head_dim, int64_t xs,
                            int64_t qs, float eps, bool mid, hipStream_t st) {
  switch (head_dim / 16) {
    case 1: return contig_launch<T, CS, NEOX, G, 1>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
    case 2: return contig_launch<T, CS, NEOX, G, 2>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
    case 4: return contig_launch<T, CS, NEOX, G, 4>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
    case 8: return contig_launch<T, CS, NEOX, G, 8>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
    default: return contig_launch<T, CS, NEOX, G, 16>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
  }
}

// Rows of 3, 5, 6 or 7 blocks of 512 channels (e.g. 24 heads of 128): heads of
// 64 or 128 only (contig_blocks), which keeps the instance count down.
template <typename T, typename CS, bool NEOX, int G>
hipError_t contig_launch_xd48(const uint16_t* x, const uint16_t* w, const void* c, const void* s,
                              uint8_t* q, float* sc, int64_t tokens, int64_t head_dim, int64_t xs,
                              int64_t qs, float eps, bool mid, hipStream_t st) {
  if (head_dim == 64) return contig_launch<T, CS, NEOX, G, 4>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
  return contig_launch<T, CS, NEOX, G, 8>(x, w, c, s, q, sc, tokens, xs, qs, eps, mid, st);
}

template <typename T, typename CS, bool NEOX>
hipError_t contig_launch_g(const uint16_t* x, const uint16_t* w, const void* c, const void* s,
                           uint8_t* q, float* sc, int64_t tokens, int64_t head_dim, int g,
                           int64_t xs, int64_t qs, float eps, bool mid, hipStream_t st) {
  switch (g) {
    case 1: return contig_launch_xd<T, CS, NEOX, 1>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 2: return contig_launch_xd<T, CS, NEOX, 2>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 3: return contig_launch_xd48<T, CS, NEOX, 3>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 4: return contig_launch_xd<T, CS, NEOX, 4>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 5: return contig_launch_xd48<T, CS, NEOX, 5>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 6: return contig_launch_xd48<T, CS, NEOX, 6>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 7: return contig_launch_xd48<T, CS, NEOX, 7>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    // two waves per token (pair_launch: heads of 64 or 128)
    case 10: return pair_launch_xd<T, CS, NEOX, 5>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 12: return pair_launch_xd<T, CS, NEOX, 6>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 14: return pair_launch_xd<T, CS, NEOX, 7>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    case 16: return pair_launch_xd<T, CS, NEOX, 8>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
    default: return contig_launch_xd<T, CS, NEOX, 8>(x, w, c, s, q, sc, tokens, head_dim, xs, qs, eps, mid, st);
  }
}

// Launch for x dtype T: cs_dtype 3 = binary32 tables, else T; neox selects
// the pairing.
template <typename T>
hipError_t contig_launch_dtype(const uint16_t* x, const uint16_t* w, const void* c,
                               const void* s, uint8_t* q, float* sc, int64_t tokens,
                               int64_t head_dim, int g, int64_t xs, int64_t qs, int cs_dtype,
                               bool neox, float eps, bool mid, hipStream_t st) {
  if (cs_dtype == 3) {
    if (neox) return contig_launch_g<T, float, true>(x, w, c, s, q, sc, tokens, head_dim, g, xs, qs, eps, mid, st);
    return contig_launch_g<T, float, false>(x, w, c, s, q, sc, tokens, head_dim, g, xs, qs, eps, mid, st);
  }
  if (neox) return contig_launch_g<T, T, true>(x, w, c, s, q, sc, tokens, head_dim, g, xs, qs, eps, mid, st);
  return contig_launch_g<T, T, false>(x, w, c, s, q, sc, tokens, head_dim, g, xs, qs, eps, mid, st);
}

}  // namespace qrw
