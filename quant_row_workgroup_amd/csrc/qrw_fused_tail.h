// qrw_fused_tail.h -- the fused RMSNorm -> RoPE -> per-token E4M3 operator
// when each head rotates only its tail span (gfx950): the kernel and its
// launch templates.  One source per x dtype (qrw_fused_tail_{bf16,f16}.hip)
// instantiates them, so the library compiles in parallel; qrw_fused_tail.hip
// holds the shape test and the dtype dispatch.
//
// Definition: "TileLang tutorial, ch. 13", s3.3.4 (RMSNorm, then RoPE on the
// tail rope_dim channels of each head, s3.3.1, then the per-token cast of
// s3.1.5); the page's own reading of its benchmark is one 4096-wide head
// rotating its last 128 channels.
//
// Mapping: the contiguous layout of the all-rotating kernel: lane l of the
// token's wave takes granules l, l+64, ..., so every load instruction covers
// 1 KiB and every code store 512 B.  Granule gi sits at position
// j = gi mod (head_dim/8) in its head and rotates when j >= s0 =
// (head_dim - rope_dim)/8.  With head_dim and rope_dim powers of two, 2*XR
// (XR = rope_dim/16) divides both 64 and s0, so a NeoX pair's partner granule
// is gi ^ XR: lane l ^ XR of the same load instruction, read with a lane
// exchange; interleaved pairs sit inside a granule.  The table granule of a
// rotated granule depends on j, hence on the load step; the table is read
// only in steps where some lane rotates (a wave-uniform test).  A lane's
// table granule is the same in every step that rotates it: a head of at most
// 64 granules sits at the same lanes in every step, and a longer head
// (rope_dim/8 <= 32 granules rotate) rotates in one step of its own, at lanes
// (s0 mod 64) and up.  So each lane reads its table granule once, with its
// row, as the all-rotating kernel does.
//
// Arithmetic as in the all-rotating kernel: z = RoPE(x * w) * rstd, amax,
// scale = max(amax, 1e-4) / 448, codes of z * (rstd / scale); with MID the
// staged form (x*w*rstd and the rotated values rounded to T, correctly
// rounded quotients of the stored values by the scale).
#pragma once

#include "qrw_contig.h"
#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

// Rows (waves) per workgroup: 4.  With the table read once, up front, 4 was
// measured fastest or within 5% of the fastest of 4, 8 and 16 (MI355X, bf16
// unless noted, outputs identical): one 4096-wide head rotating its last 128
// channels at 1024 / 2048 / 4096 / 8192 / 16384 tokens 5.09 / 7.04 / 10.86 /
// 19.31 / 35.35 us against 7.95 / 8.98 / 11.63 / 21.77 / 39.67 us at 16 rows;
// 32 heads of 128 rotating 64 at 1024 / 4096 / 16384 tokens 5.72 / 11.93 /
// 36.87 us against 8.68 / 11.90 / 42.85 us.  (16-row workgroups are ahead only
// where they fill the GPU in exactly one round, 4096 tokens: by 1-5%.)
constexpr int kTailRows = 4;

// PACKED: the codes' row stride is x's (a packed call), one stride for both,
// as in the all-rotating kernel.
// PAIR: the row is 2 * G blocks, and two waves of the workgroup take one half
// each (kTailRows / 2 tokens per workgroup), exchanging the sum of squares and
// the amax through LDS behind one workgroup barrier each, as the all-rotating
// kernel's pair form does; a head of at most 64 granules sits at the same
// lanes in both halves (G * 64 granules is a multiple of it), so the span test
// and the table granule are the same.  Every wave reaches both barriers: a
// token past the end touches no memory.
template <typename T, typename CS, bool NEOX, int G, bool HAS_W, int XR, bool MID, bool PACKED,
          bool PAIR = false>
__global__ __launch_bounds__(kWave * kTailRows) void rmsnorm_rope_fp8_tail_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const void* cosv, const void* sinv,
    uint8_t* q, float* scales, int64_t tokens, int64_t xs, int64_t qs, int half, int hg_mask,
    int s0, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int64_t t = PAIR ? (int64_t)blockIdx.x * (kTailRows / 2) + (wv >> 1)
                         : (int64_t)blockIdx.x * kTailRows + wv;
  const int part = PAIR ? (wv & 1) : 0;  // which half of the row (PAIR)
  const bool live = t < tokens;
  if (!PAIR && !live) return;  // wave-uniform
  const int64_t c0 = (int64_t)part * (512 * G);  // first channel of this wave's part
  const uint16_t* xr = x + t * xs + c0;
  uint8_t* qr = q + t * (PACKED ? xs : qs) + c0;
  if (PAIR && HAS_W) w += c0;

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
  // this lane's position in the rotated span in the steps that rotate it
  // (< 0: none; its table granule is then a valid, unused one)
  const int jl = contig_span_pos(lane, hg_mask, s0);
  // (a token past the end reads token 0's rows, which exist when a kernel runs)
  const char* crow = table_row<CS>(cosv, live ? t : 0, half);
  const char* srow = table_row<CS>(sinv, live ? t : 0, half);
  float c[8], sn[8];
  if (NEOX) {
    const int tg = jl >= 0 ? (jl & (XR - 1)) : 0;
    Table8<CS>::load(crow, tg, c);
    Table8<CS>::load(srow, tg, sn);
    if (jl < XR) {  // first half of the span: x c - x_partner s
#pragma unroll
      for (int e = 0; e < 8; ++e) sn[e] = -sn[e];
    }
  } else {
    float c4[4], s4[4];
    Table4<CS>::load(crow, jl >= 0 ? jl : 0, c4);
    Table4<CS>::load(srow, jl >= 0 ? jl : 0, s4);
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
  __shared__ float pair_slot[kTailRows / 2][4];  // PAIR: [part] sums, [2 + part] maxima
  if constexpr (PAIR) {
    if (lane == 0) pair_slot[wv >> 1][part] = ss;
    __syncthreads();
    ss = pair_slot[wv >> 1][0] + pair_slot[wv >> 1][1];
  }
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
    if (MID) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[g][e] *= rstd;
      round8<T>(v[g]);
    }
    // this step rotates the lane when its granule is in the span (then at
    // position jl)
    const bool span = contig_rotates(kWave * g + lane, hg_mask, s0);
    if (__builtin_amdgcn_ballot_w64(span) != 0) {  // wave-uniform: some lane rotates
      if (NEOX) {
        float rv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rv[e] = fmaf(v[g][e], c[e], lane_xor<XR>(v[g][e]) * sn[e]);
        if (span) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[g][e] = rv[e];
        }
      } else if (span) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = v[g][2 * k], x1 = v[g][2 * k + 1];
          v[g][2 * k] = fmaf(x0, c[k], -(x1 * sn[k]));
          v[g][2 * k + 1] = fmaf(x1, c[k], x0 * sn[k]);
        }
      }
      if (MID) round8<T>(v[g]);  // unrotated values are already T values
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      m[(e >> 1) & 3] = fmaxf(m[(e >> 1) & 3], fmaxf(fabsf(v[g][e]), fabsf(v[g][e + 1])));
  }
  const float amax = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  float amax_w = wave_max(amax);
  if constexpr (PAIR) {
    if (lane == 0) pair_slot[wv >> 1][2 + part] = amax_w;
    __syncthreads();
    amax_w = fmaxf(pair_slot[wv >> 1][2], pair_slot[wv >> 1][3]);
  }
  const float amax_z = MID ? amax_w : amax_w * rstd;
  const float scale = scale_e4m3(fmaxf(amax_z, 1e-4f));
  const float kq = rstd / scale;
  const float inv = recip_rn(scale);
  if (lane == 0 && (!PAIR || (live && part == 0))) scales[t] = scale;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = MID ? div_rn(v[g][e], scale, inv) : v[g][e] * kq;
    if (PAIR && !live) continue;
    st8(qr + 8 * (kWave * g + lane), fp8x8(a));
  }
}

// ------------------------------------------------------------------ launch
template <typename T, typename CS, bool NEOX, int G, int XR, bool PAIR = false>
void tail_go(dim3 grid, hipStream_t st, const void* x, const void* w, const void* c,
             const void* s, uint8_t* q, float* sc, int64_t tokens, int64_t xs, int64_t qs,
             int half, int hg_mask, int s0, float eps, bool mid) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  if (PAIR) grid = dim3((unsigned)((tokens + kTailRows / 2 - 1) / (kTailRows / 2)));
#define QRW_TAIL_LAUNCH(HW, M, P)                                                                  \
  rmsnorm_rope_fp8_tail_kernel<T, CS, NEOX, G, HW, XR, M, P, PAIR><<<grid, kWave * kTailRows, 0, st>>>( \
      xp, wp, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps)
  // the packed instances are the weighted ones (the usual call)
  const bool packed = qs == xs;
  if (mid) {
    if (wp && packed) QRW_TAIL_LAUNCH(true, true, true);
    else if (wp) QRW_TAIL_LAUNCH(true, true, false);
    else QRW_TAIL_LAUNCH(false, true, false);
  } else {
    if (wp && packed) QRW_TAIL_LAUNCH(true, false, true);
    else if (wp) QRW_TAIL_LAUNCH(true, false, false);
    else QRW_TAIL_LAUNCH(false, false, false);
  }
#undef QRW_TAIL_LAUNCH
}

template <typename T, typename CS, bool NEOX, int G>
void tail_go_xr(int xr, dim3 grid, hipStream_t st, const void* x, const void* w, const void* c,
                const void* s, uint8_t* q, float* sc, int64_t tokens, int64_t xs, int64_t qs,
                int half, int hg_mask, int s0, float eps, bool mid) {
  if constexpr (!NEOX) {
    tail_go<T, CS, NEOX, G, 1>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid);
  } else {
    switch (xr) {
      case 1: tail_go<T, CS, NEOX, G, 1>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      case 2: tail_go<T, CS, NEOX, G, 2>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      case 4: tail_go<T, CS, NEOX, G, 4>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      case 8: tail_go<T, CS, NEOX, G, 8>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      default: tail_go<T, CS, NEOX, G, 16>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    }
  }
}

// Rows of 3, 5, 6 or 7 blocks: heads of 64 or 128 (fused_tail_ok), so the span
// is at most 64 channels and rope_dim / 16 is 1, 2 or 4; this keeps the
// instance count down.
template <typename T, typename CS, bool NEOX, int G>
void tail_go_xr124(int xr, dim3 grid, hipStream_t st, const void* x, const void* w,
                   const void* c, const void* s, uint8_t* q, float* sc, int64_t tokens,
                   int64_t xs, int64_t qs, int half, int hg_mask, int s0, float eps, bool mid) {
  if constexpr (!NEOX) {
    tail_go<T, CS, NEOX, G, 1>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid);
  } else {
    switch (xr) {
      case 1: tail_go<T, CS, NEOX, G, 1>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      case 2: tail_go<T, CS, NEOX, G, 2>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      default: tail_go<T, CS, NEOX, G, 4>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    }
  }
}

// Rows of 10, 12, 14 or 16 blocks, heads of 64 or 128: two waves per token,
// each on G = 5 ... 8 blocks.
template <typename T, typename CS, bool NEOX, int G>
void tail_go_pair(int xr, dim3 grid, hipStream_t st, const void* x, const void* w,
                  const void* c, const void* s, uint8_t* q, float* sc, int64_t tokens,
                  int64_t xs, int64_t qs, int half, int hg_mask, int s0, float eps, bool mid) {
  if constexpr (!NEOX) {
    tail_go<T, CS, NEOX, G, 1, true>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid);
  } else {
    switch (xr) {
      case 1: tail_go<T, CS, NEOX, G, 1, true>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      case 2: tail_go<T, CS, NEOX, G, 2, true>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
      default: tail_go<T, CS, NEOX, G, 4, true>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    }
  }
}

template <typename T, typename CS, bool NEOX>
void tail_go_g(int gg, int xr, dim3 grid, hipStream_t st, const void* x, const void* w,
               const void* c, const void* s, uint8_t* q, float* sc, int64_t tokens, int64_t xs,
               int64_t qs, int half, int hg_mask, int s0, float eps, bool mid) {
  switch (gg) {
    case 1: tail_go_xr<T, CS, NEOX, 1>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 2: tail_go_xr<T, CS, NEOX, 2>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 3: tail_go_xr124<T, CS, NEOX, 3>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 4: tail_go_xr<T, CS, NEOX, 4>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 5: tail_go_xr124<T, CS, NEOX, 5>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 6: tail_go_xr124<T, CS, NEOX, 6>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 7: tail_go_xr124<T, CS, NEOX, 7>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 10: tail_go_pair<T, CS, NEOX, 5>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 12: tail_go_pair<T, CS, NEOX, 6>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 14: tail_go_pair<T, CS, NEOX, 7>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    case 16: tail_go_pair<T, CS, NEOX, 8>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
    default: tail_go_xr<T, CS, NEOX, 8>(xr, grid, st, x, w, c, s, q, sc, tokens, xs, qs, half, hg_mask, s0, eps, mid); break;
  }
}

// All tail kernels of x dtype T: cs_dtype 3 = binary32 tables, else T.
template <typename T>
hipError_t tail_launch_dtype(const void* x, const void* w, const void* cos, const void* sin,
                             uint8_t* q, float* scales, int64_t tokens, int64_t heads,
                             int64_t head_dim, int64_t rope_dim, int64_t xs, int64_t qs,
                             int cs_dtype, bool neox, float eps, bool round_mid,
                             hipStream_t stream) {
  const dim3 grid((unsigned)((tokens + kTailRows - 1) / kTailRows));
  const int gg = (int)(heads * head_dim / 512);
  const int xr = (int)(rope_dim / 16);
  const int half = (int)(rope_dim / 2);
  const int hg_mask = (int)(head_dim / 8 - 1);
  const int s0 = (int)((head_dim - rope_dim) / 8);
#define QRW_TAIL_ARGS gg, xr, grid, stream, x, w, cos, sin, q, scales, tokens, xs, qs, half, \
                      hg_mask, s0, eps, round_mid
  if (cs_dtype == 3) {
    if (neox) tail_go_g<T, float, true>(QRW_TAIL_ARGS);
    else tail_go_g<T, float, false>(QRW_TAIL_ARGS);
  } else {
    if (neox) tail_go_g<T, T, true>(QRW_TAIL_ARGS);
    else tail_go_g<T, T, false>(QRW_TAIL_ARGS);
  }
#undef QRW_TAIL_ARGS
  return hipGetLastError();
}

// One per x dtype, each in its own source.
hipError_t launch_rmsnorm_rope_fp8_tail_bf16(const void* x, const void* w, const void* cos,
                                             const void* sin, uint8_t* q, float* scales,
                                             int64_t tokens, int64_t heads, int64_t head_dim,
                                             int64_t rope_dim, int64_t xs, int64_t qs,
                                             int cs_dtype, bool neox, float eps, bool round_mid,
                                             hipStream_t stream);
hipError_t launch_rmsnorm_rope_fp8_tail_f16(const void* x, const void* w, const void* cos,
                                            const void* sin, uint8_t* q, float* scales,
                                            int64_t tokens, int64_t heads, int64_t head_dim,
                                            int64_t rope_dim, int64_t xs, int64_t qs,
                                            int cs_dtype, bool neox, float eps, bool round_mid,
                                            hipStream_t stream);



}  // namespace qrw
