// qrw_rope.hip -- RoPE (interleaved and NeoX half-split) and the fused
// RMSNorm -> RoPE -> per-token FP8 kernel (gfx950).
//
// Definitions: "TileLang tutorial, ch. 13": the pairings and the cos/sin table
// of shape (positions, rope_dim/2) in s3.3.1; the reference RoPE (binary32
// math, a single final cast) in s3.3.2; the fused operator in s3.3.4; the
// per-token cast (amax -> scale = max(amax, 1e-4)/fp8_max -> clamp -> cast)
// in s3.1.5.
//
// RoPE shapes with power-of-two heads and rows of 512 * {1, 2, 4, 8, 16}
// channels take the contiguous kernel (qrw_rope_contig.hip); the item kernel
// below serves every other shape.
//
// Mapping: one wave64 per token, four tokens per workgroup.  The token row is
// cut into items of two granules (qrw_plan.h) such that both channels of every
// rotation pair sit in the same lane, so the rotation needs no LDS and no
// cross-lane exchange -- the pairing the page routes through shared memory
// is lane-local here.  A lane first issues the loads of all of its items, then
// computes, then stores.  When rope_dim/16 divides 64, each lane only ever
// needs one 8-entry granule of the token's cos/sin row, loaded once.
//
// Cache hints (measured on MI355X at the benchmark sizes): x is read with
// non-temporal loads everywhere; RoPE also writes y non-temporally, while the
// fused kernel's FP8 codes are stored normally (faster there).
//
// Fused arithmetic (binary32).  Because RoPE is linear and rstd is a per-row
// scalar, the kernel evaluates z = RoPE(x * w) * rstd: u = x * w is exact in
// binary32 for 16-bit operands, the rotation rounds once per output (fma),
// and the quantiser multiplies by k = rstd / scale.  amax is taken over
// |RoPE(x * w)| and scaled by rstd once per row.  With this order every code
// satisfies |z * k| <= 448 * (1 + 4 * 2^-24) < 464, so the round-to-nearest
// E4M3 conversion never leaves the finite range and the clamp of s3.1.5 is a
// no-op that is not executed.
#include <type_traits>

#include "qrw_device.h"
#include "qrw_launch.h"
#include "qrw_plan.h"

namespace qrw {

// Rotate one item in place.  NeoX: channel e of A pairs with channel e of B,
// using table entry e.  Interleaved: channels (2k, 2k+1) of A use entry k and
// those of B use entry 4 + k.  First of a pair: x_a c - x_b s; second:
// x_a s + x_b c.
template <bool NEOX>
__device__ __forceinline__ void rotate(float (&a)[8], float (&b)[8], const float (&c)[8],
                                       const float (&s)[8]) {
  if (NEOX) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xa = a[e], xb = b[e];
      a[e] = fmaf(xa, c[e], -(xb * s[e]));
      b[e] = fmaf(xb, c[e], xa * s[e]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x0 = a[2 * k], x1 = a[2 * k + 1];
      a[2 * k] = fmaf(x0, c[k], -(x1 * s[k]));
      a[2 * k + 1] = fmaf(x1, c[k], x0 * s[k]);
      x0 = b[2 * k];
      x1 = b[2 * k + 1];
      b[2 * k] = fmaf(x0, c[4 + k], -(x1 * s[4 + k]));
      b[2 * k + 1] = fmaf(x1, c[4 + k], x0 * s[4 + k]);
    }
  }
}

// ------------------------------------------------------------------ RoPE
template <typename T, typename CS, bool NEOX, int K>
__global__ __launch_bounds__(kBlock) void rope_kernel(const uint16_t* x, const void* cosv,
                                                      const void* sinv, uint16_t* y,
                                                      int64_t tokens, int64_t xs, int64_t ys,
                                                      RowPlan pl, int copy_plain) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const uint16_t* xr = x + t * xs;
  uint16_t* yr = y + t * ys;
  const char* crow = table_row<CS>(cosv, t, pl.half);
  const char* srow = table_row<CS>(sinv, t, pl.half);

  float hc[8], hs[8];
  if (pl.lane_hoist) {
    const int s0 = lane % pl.gph;
    Table8<CS>::load(crow, s0, hc);
    Table8<CS>::load(srow, s0, hs);
  }

  for (int base = 0; base < pl.n_items; base += kWave * K) {
    int kind[K], oa[K], ob[K], si[K];
    u32x4 ra[K], rb[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      kind[i] = item_offsets(pl, base + lane + kWave * i, NEOX, oa[i], ob[i], si[i]);
      if (kind[i] == kItemPlain && !copy_plain) kind[i] = kItemNone;
      ra[i] = (u32x4){0u, 0u, 0u, 0u};
      rb[i] = (u32x4){0u, 0u, 0u, 0u};
      if (kind[i] != kItemNone) ra[i] = ld16_stream(xr + oa[i]);
      if (kind[i] != kItemNone && ob[i] >= 0) rb[i] = ld16_stream(xr + ob[i]);
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (kind[i] == kItemRope) {
        float c[8], s[8], a[8], b[8];
        if (pl.lane_hoist) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            c[e] = hc[e];
            s[e] = hs[e];
          }
        } else {
          Table8<CS>::load(crow, si[i], c);
          Table8<CS>::load(srow, si[i], s);
        }
        widen8<T>(ra[i], a);
        widen8<T>(rb[i], b);
        rotate<NEOX>(a, b, c, s);
        st16_stream(yr + oa[i], narrow8<T>(a));
        st16_stream(yr + ob[i], narrow8<T>(b));
      } else if (kind[i] == kItemPlain) {
        st16_stream(yr + oa[i], ra[i]);
        if (ob[i] >= 0) st16_stream(yr + ob[i], rb[i]);
      }
    }
  }
}

// ------------------------------------------------------------------ fused
// MID: the staged form of the page's fused dataflow, which writes the
// normalised row back to shared memory in x's dtype and rotates it there: the
// normalised values x * rstd * w and the rotated values are each rounded to
// T, and the codes quantise those stored values: the composition of the three
// operators, up to the 16-bit neighbour chosen where an exact intermediate is
// within the binary32 evaluation's error of a rounding boundary.  Without MID
// the row stays in binary32 from the load to the codes.
template <typename T, typename CS, bool NEOX, int K, bool MID>
__global__ __launch_bounds__(kBlock) void rmsnorm_rope_fp8_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const void* cosv, const void* sinv,
    uint8_t* q, float* scales, int64_t tokens, int64_t xs, int64_t qs, RowPlan pl, float n_f,
    float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= tokens) return;
  const uint16_t* xr = x + t * xs;
  uint8_t* qr = q + t * qs;
  const char* crow = table_row<CS>(cosv, t, pl.half);
  const char* srow = table_row<CS>(sinv, t, pl.half);

  // 1. issue the loads of every granule this lane owns
  int kind[K], oa[K], ob[K], si[K];
  u32x4 ra[K], rb[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    kind[i] = item_offsets(pl, lane + kWave * i, NEOX, oa[i], ob[i], si[i]);
    ra[i] = (u32x4){0u, 0u, 0u, 0u};
    rb[i] = (u32x4){0u, 0u, 0u, 0u};
    if (kind[i] != kItemNone) ra[i] = ld16_stream(xr + oa[i]);
    if (kind[i] != kItemNone && ob[i] >= 0) rb[i] = ld16_stream(xr + ob[i]);
  }
  float hc[8], hs[8];
  if (pl.lane_hoist) {
    const int s0 = lane % pl.gph;
    Table8<CS>::load(crow, s0, hc);
    Table8<CS>::load(srow, s0, hs);
  }

  // 2. RMS statistics (absent granules are zero and add nothing)
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < K; ++i) {
    float a[8], b[8];
    widen8<T>(ra[i], a);
    widen8<T>(rb[i], b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] = fmaf(a[e], a[e], acc[e]);
      acc[e] = fmaf(b[e], b[e], acc[e]);
    }
  }
  const float ss = wave_sum(tree8(acc));
  const float rstd = 1.0f / sqrtf(ss / n_f + eps);

  // 3. v = RoPE(x * w), kept in registers; running max |v|
  float va[K][8], vb[K][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    widen8<T>(ra[i], va[i]);
    widen8<T>(rb[i], vb[i]);
    if (w) {
      float wa[8], wb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wa[e] = 0.0f;
        wb[e] = 0.0f;
      }
      if (kind[i] != kItemNone) widen8<T>(ld16(w + oa[i]), wa);
      if (kind[i] != kItemNone && ob[i] >= 0) widen8<T>(ld16(w + ob[i]), wb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        va[i][e] *= wa[e];
        vb[i][e] *= wb[e];
      }
    }
    if (MID) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        va[i][e] *= rstd;
        vb[i][e] *= rstd;
      }
      round8<T>(va[i]);
      round8<T>(vb[i]);
    }
    if (kind[i] == kItemRope) {
      float c[8], s[8];
      if (pl.lane_hoist) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          c[e] = hc[e];
          s[e] = hs[e];
        }
      } else {
        Table8<CS>::load(crow, si[i], c);
        Table8<CS>::load(srow, si[i], s);
      }
      rotate<NEOX>(va[i], vb[i], c, s);
      if (MID) {
        round8<T>(va[i]);
        round8<T>(vb[i]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fmaxf(fabsf(va[i][e]), fabsf(vb[i][e])));
  }

  // 4. per-token scale (s3.1.5): scale = max(amax_z, 1e-4) / 448, amax_z = amax * rstd
  //    (MID: the stored values already carry rstd)
  const float amax_z = MID ? wave_max(amax) : wave_max(amax) * rstd;
  const float scale = scale_e4m3(fmaxf(amax_z, 1e-4f));
  const float k = rstd / scale;
  const float inv = recip_rn(scale);
  if (lane == 0) scales[t] = scale;

  // 5. quantise and store the codes
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (kind[i] != kItemNone) {
      float a[8], b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // MID: the correctly rounded quotient of the stored value, as the
        // standalone per-token cast forms it
        a[e] = MID ? div_rn(va[i][e], scale, inv) : va[i][e] * k;
        b[e] = MID ? div_rn(vb[i][e], scale, inv) : vb[i][e] * k;
      }
      st8(qr + oa[i], fp8x8(a));
      if (ob[i] >= 0) st8(qr + ob[i], fp8x8(b));
    }
  }
}


// ------------------------------------------------------------------ fused, dense
// The same operator when every lane owns exactly K rope items and a single
// table granule: no pass-through channels, rope_dim/16 a power of two that
// divides 64, and heads * rope_dim/16 == 64 * K (e.g. 32 heads x 128 with
// K = 4).  Offsets are closed-form and nothing is predicated; the sum of
// squares runs on the packed pairs with v_dot2c.
//
// Each wave handles RPW tokens (kDenseRpw), t = wave, wave + W, ... (W waves
// in the grid), software-pipelined when RPW > 1: the loads of token k+1 are issued as soon as
// token k's data is in registers, before token k is computed and stored, so
// reads of later tokens overlap the arithmetic and the stores of earlier ones
// instead of every wave waiting for the last of all reads.  The weight
// granules are loaded once per wave and reused for all of its tokens.
template <typename T, typename CS, bool NEOX, int K, bool HAS_W>
__device__ __forceinline__ void dense_token(const u32x4 (&ra)[K], const u32x4 (&rb)[K],
                                            const u32x4 (&wa)[K], const u32x4 (&wb)[K],
                                            const float (&c)[8], const float (&sn)[8],
                                            const int (&oa)[K], int bo, uint8_t* qr,
                                            float* scale_out, int lane, float n_f, float eps) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < K; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[k] = sumsq2(T{}, ra[i][k], acc[k]);
      acc[4 + k] = sumsq2(T{}, rb[i][k], acc[4 + k]);
    }
  }
  const float ss = wave_sum(tree8(acc));
  const float rstd = 1.0f / sqrtf(ss / n_f + eps);

  float va[K][8], vb[K][8];
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < K; ++i) {
    widen8<T>(ra[i], va[i]);
    widen8<T>(rb[i], vb[i]);
    if (HAS_W) {
      float fa[8], fb[8];
      widen8<T>(wa[i], fa);
      widen8<T>(wb[i], fb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        va[i][e] *= fa[e];
        vb[i][e] *= fb[e];
      }
    }
    rotate<NEOX>(va[i], vb[i], c, sn);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      m[e & 3] = fmaxf(m[e & 3], fmaxf(fabsf(va[i][e]), fabsf(vb[i][e])));
  }
  const float amax = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  const float amax_z = wave_max(amax) * rstd;
  const float scale = scale_e4m3(fmaxf(amax_z, 1e-4f));
  const float kq = rstd / scale;
  if (lane == 0) *scale_out = scale;

#pragma unroll
  for (int i = 0; i < K; ++i) {
    float a[8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = va[i][e] * kq;
      b[e] = vb[i][e] * kq;
    }
    const u32x2 ca = fp8x8(a), cb = fp8x8(b);
    if (NEOX) {
      st8(qr + oa[i], ca);
      st8(qr + oa[i] + bo, cb);
    } else {
      st16(qr + oa[i], (u32x4){ca[0], ca[1], cb[0], cb[1]});
    }
  }
}

template <typename T, typename CS, bool NEOX, int K, bool HAS_W, int RPW>
__global__ __launch_bounds__(kBlock) void rmsnorm_rope_fp8_dense_kernel(
    const uint16_t* x, const uint16_t* __restrict__ w, const void* cosv, const void* sinv,
    uint8_t* q, float* scales, int64_t tokens, int64_t xs, int64_t qs, int head_dim,
    int half, int lg_gph, float n_f, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kRowsPerBlock;
  if (wave >= tokens) return;  // wave-uniform; later tokens of this wave are further out
  const int s = lane & ((1 << lg_gph) - 1);
  const int bo = NEOX ? half : 8;  // B granule offset from A

  int oa[K];
#pragma unroll
  for (int i = 0; i < K; ++i)
    oa[i] = ((lane + kWave * i) >> lg_gph) * head_dim + (NEOX ? 8 * s : 16 * s);

  u32x4 wa[K], wb[K];
  if (HAS_W) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      wa[i] = ld16(w + oa[i]);
      wb[i] = ld16(w + oa[i] + bo);
    }
  }

  // token `wave`: loads
  int64_t t = wave;
  u32x4 ra[K], rb[K];
  {
    const uint16_t* xr = x + t * xs;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      ra[i] = ld16_stream(xr + oa[i]);
      rb[i] = ld16_stream(xr + oa[i] + bo);
    }
  }
  float c[8], sn[8];
  Table8<CS>::load(table_row<CS>(cosv, t, half), s, c);
  Table8<CS>::load(table_row<CS>(sinv, t, half), s, sn);

#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int64_t tn = t + nwaves;
    const bool more = (r + 1 < RPW) && tn < tokens;  // wave-uniform
    u32x4 na[K], nb[K];
    float nc[8], ns[8];
    if (r + 1 < RPW) {
      // Issue the next token's loads before this token's arithmetic.  They are
      // unconditional (a past-the-end token reloads the last one) so that the
      // wait for this token's data does not also wait for them.
      const int64_t tl = more ? tn : tokens - 1;
      const uint16_t* xn = x + tl * xs;
#pragma unroll
      for (int i = 0; i < K; ++i) {
        na[i] = ld16_stream(xn + oa[i]);
        nb[i] = ld16_stream(xn + oa[i] + bo);
      }
      Table8<CS>::load(table_row<CS>(cosv, tl, half), s, nc);
      Table8<CS>::load(table_row<CS>(sinv, tl, half), s, ns);
    }
    dense_token<T, CS, NEOX, K, HAS_W>(ra, rb, wa, wb, c, sn, oa, bo, q + t * qs, scales + t,
                                       lane, n_f, eps);
    if (!more) break;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      ra[i] = na[i];
      rb[i] = nb[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      c[e] = nc[e];
      sn[e] = ns[e];
    }
    t = tn;
  }
}

// ------------------------------------------------------------------ launch
int64_t fused_items(int64_t heads, int64_t head_dim, int64_t rope_dim) {
  return make_plan(heads, head_dim, rope_dim).n_items;
}

namespace {

template <typename T, typename CS, bool NEOX>
void rope_go(int kk, dim3 grid, hipStream_t st, const uint16_t* x, const void* c, const void* s,
             uint16_t* y, int64_t tokens, int64_t xs, int64_t ys, const RowPlan& pl, int copy) {
  switch (kk) {
    case 1: rope_kernel<T, CS, NEOX, 1><<<grid, kBlock, 0, st>>>(x, c, s, y, tokens, xs, ys, pl, copy); break;
    case 2: rope_kernel<T, CS, NEOX, 2><<<grid, kBlock, 0, st>>>(x, c, s, y, tokens, xs, ys, pl, copy); break;
    default: rope_kernel<T, CS, NEOX, 4><<<grid, kBlock, 0, st>>>(x, c, s, y, tokens, xs, ys, pl, copy); break;
  }
}

template <typename T, typename CS>
void rope_go2(bool neox, int kk, dim3 grid, hipStream_t st, const uint16_t* x, const void* c,
              const void* s, uint16_t* y, int64_t tokens, int64_t xs, int64_t ys,
              const RowPlan& pl, int copy) {
  if (neox) rope_go<T, CS, true>(kk, grid, st, x, c, s, y, tokens, xs, ys, pl, copy);
  else rope_go<T, CS, false>(kk, grid, st, x, c, s, y, tokens, xs, ys, pl, copy);
}

// Tokens per wave of the dense kernel.  1: pipelining several tokens per wave
// did not pay at these sizes on MI355X (the kernel keeps the capability).
constexpr int kDenseRpw = 1;

template <typename T, typename CS, bool NEOX, int K>
void dense_go(dim3 grid, hipStream_t st, const uint16_t* x, const uint16_t* w, const void* c,
              const void* s, uint8_t* q, float* sc, int64_t tokens, int64_t xs, int64_t qs,
              const RowPlan& pl, float n_f, float eps) {
  constexpr int kRpw = kDenseRpw;
  int lg = 0;
  while ((1 << lg) < pl.gph) ++lg;
  const dim3 g((unsigned)((tokens + (int64_t)kRowsPerBlock * kRpw - 1) /
                          ((int64_t)kRowsPerBlock * kRpw)));
  (void)grid;
  if (w)
    rmsnorm_rope_fp8_dense_kernel<T, CS, NEOX, K, true, kRpw><<<g, kBlock, 0, st>>>(
        x, w, c, s, q, sc, tokens, xs, qs, pl.head_dim, pl.half, lg, n_f, eps);
  else
    rmsnorm_rope_fp8_dense_kernel<T, CS, NEOX, K, false, kRpw><<<g, kBlock, 0, st>>>(
        x, w, c, s, q, sc, tokens, xs, qs, pl.head_dim, pl.half, lg, n_f, eps);
}

// The dense path applies when every lane owns exactly K rope items that all
// use the lane's one table granule (see rmsnorm_rope_fp8_dense_kernel).
bool dense_ok(const RowPlan& pl, int kk) {
  const bool pow2 = (pl.gph & (pl.gph - 1)) == 0;
  return pl.n_plain == 0 && pl.lane_hoist && pow2 && pl.n_rope == kWave * kk;
}

// Granules per lane of the contiguous path, or 0 if it does not apply: whole
// heads rotate, head_dim / 16 is 1, 2, 4, 8 or 16, and the row is 1, 2, 4 or
// 8 blocks of 512 channels -- or 3, 5, 6, 7 blocks of heads of 64 or 128, or
// 10, 12, 14, 16 blocks of them (two waves per token).
int contig_blocks(const RowPlan& pl) {
  const int xd = pl.head_dim / 16;
  const bool xd_ok = pl.head_dim % 16 == 0 && (xd == 1 || xd == 2 || xd == 4 || xd == 8 || xd == 16);
  if (pl.pass != 0 || !xd_ok || pl.n % 512 != 0) return 0;
  const int g = pl.n / 512;
  if (g == 1 || g == 2 || g == 4 || g == 8) return g;
  const bool odd_ok = pl.head_dim == 64 || pl.head_dim == 128;
  return odd_ok && (g == 3 || g == 5 || g == 6 || g == 7 || g == 10 || g == 12 || g == 14 ||
                    g == 16) ? g : 0;
}

template <typename T, typename CS, bool NEOX>
void fused_go(int kk, dim3 grid, hipStream_t st, const uint16_t* x, const uint16_t* w,
              const void* c, const void* s, uint8_t* q, float* sc, int64_t tokens, int64_t xs,
              int64_t qs, const RowPlan& pl, float n_f, float eps, bool mid) {
  if (mid) {  // the staged form on any other shape: the item kernel
    switch (kk) {
      case 1: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 1, true><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
      case 2: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 2, true><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
      case 4: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 4, true><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
      default: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 8, true><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
    }
    return;
  }
  if (dense_ok(pl, kk)) {
    switch (kk) {
      case 1: dense_go<T, CS, NEOX, 1>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); return;
      case 2: dense_go<T, CS, NEOX, 2>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); return;
      case 4: dense_go<T, CS, NEOX, 4>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); return;
      default: dense_go<T, CS, NEOX, 8>(grid, st, x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); return;
    }
  }
  switch (kk) {
    case 1: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 1, false><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
    case 2: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 2, false><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
    case 4: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 4, false><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
    default: rmsnorm_rope_fp8_kernel<T, CS, NEOX, 8, false><<<grid, kBlock, 0, st>>>(x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps); break;
  }
}

template <typename T, typename CS>
void fused_go2(bool neox, int kk, dim3 grid, hipStream_t st, const uint16_t* x,
               const uint16_t* w, const void* c, const void* s, uint8_t* q, float* sc,
               int64_t tokens, int64_t xs, int64_t qs, const RowPlan& pl, float n_f,
               float eps, bool mid) {
  if (neox) fused_go<T, CS, true>(kk, grid, st, x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps, mid);
  else fused_go<T, CS, false>(kk, grid, st, x, w, c, s, q, sc, tokens, xs, qs, pl, n_f, eps, mid);
}

int items_per_lane(int n_items, int kmax) {
  int k = 1;
  while (k < kmax && k * kWave < n_items) k *= 2;
  return k;
}

}  // namespace

hipError_t launch_rope(const void* x, const void* cos, const void* sin, void* y, int64_t tokens,
                       int64_t heads, int64_t head_dim, int64_t rope_dim, int64_t xs,
                       int64_t ys, int dtype, int cs_dtype, bool neox, hipStream_t stream) {
  if (rope_contig_ok(heads, head_dim, rope_dim, neox))
    return launch_rope_contig(x, cos, sin, y, tokens, heads, head_dim, rope_dim, xs, ys, dtype,
                              cs_dtype, neox, stream);
  const RowPlan pl = make_plan(heads, head_dim, rope_dim);
  const int kk = items_per_lane(pl.n_items, 4);
  const dim3 grid((unsigned)((tokens + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto* xp = static_cast<const uint16_t*>(x);
  auto* yp = static_cast<uint16_t*>(y);
  const int copy = (x != y) ? 1 : 0;  // in place: pass-through channels are already there
  if (dtype == 1) {
    if (cs_dtype == 3) rope_go2<F16, float>(neox, kk, grid, stream, xp, cos, sin, yp, tokens, xs, ys, pl, copy);
    else rope_go2<F16, F16>(neox, kk, grid, stream, xp, cos, sin, yp, tokens, xs, ys, pl, copy);
  } else {
    if (cs_dtype == 3) rope_go2<BF16, float>(neox, kk, grid, stream, xp, cos, sin, yp, tokens, xs, ys, pl, copy);
    else rope_go2<BF16, BF16>(neox, kk, grid, stream, xp, cos, sin, yp, tokens, xs, ys, pl, copy);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rope_fp8(const void* x, const void* w, const void* cos,
                                   const void* sin, uint8_t* q, float* scales, int64_t tokens,
                                   int64_t heads, int64_t head_dim, int64_t rope_dim,
                                   int64_t xs, int64_t qs, int dtype, int cs_dtype, bool neox,
                                   float eps, bool round_mid, hipStream_t stream) {
  const RowPlan pl = make_plan(heads, head_dim, rope_dim);
  const int g = contig_blocks(pl);
  if (g != 0) {
    const auto* xp = static_cast<const uint16_t*>(x);
    const auto* wp = static_cast<const uint16_t*>(w);
    if (dtype == 1)
      return launch_rmsnorm_rope_fp8_contig_f16(xp, wp, cos, sin, q, scales, tokens, head_dim, g,
                                                xs, qs, cs_dtype, neox, eps, round_mid, stream);
    return launch_rmsnorm_rope_fp8_contig_bf16(xp, wp, cos, sin, q, scales, tokens, head_dim, g,
                                               xs, qs, cs_dtype, neox, eps, round_mid, stream);
  }
  if (fused_tail_ok(heads, head_dim, rope_dim))
    return launch_rmsnorm_rope_fp8_tail(x, w, cos, sin, q, scales, tokens, heads, head_dim,
                                        rope_dim, xs, qs, dtype, cs_dtype, neox, eps, round_mid,
                                        stream);
  const int kk = items_per_lane(pl.n_items, 8);
  const dim3 grid((unsigned)((tokens + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w);
  const float n_f = (float)pl.n;
  if (dtype == 1) {
    if (cs_dtype == 3) fused_go2<F16, float>(neox, kk, grid, stream, xp, wp, cos, sin, q, scales, tokens, xs, qs, pl, n_f, eps, round_mid);
    else fused_go2<F16, F16>(neox, kk, grid, stream, xp, wp, cos, sin, q, scales, tokens, xs, qs, pl, n_f, eps, round_mid);
  } else {
    if (cs_dtype == 3) fused_go2<BF16, float>(neox, kk, grid, stream, xp, wp, cos, sin, q, scales, tokens, xs, qs, pl, n_f, eps, round_mid);
    else fused_go2<BF16, BF16>(neox, kk, grid, stream, xp, wp, cos, sin, q, scales, tokens, xs, qs, pl, n_f, eps, round_mid);
  }
  return hipGetLastError();
}

}  // namespace qrw
