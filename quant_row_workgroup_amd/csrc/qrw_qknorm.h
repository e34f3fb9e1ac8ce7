// qrw_qknorm.h -- per-head QK RMSNorm + RoPE, in place on a packed QKV row
// (gfx950): the kernel template and its type dispatch.  Each chunk width GC
// is instantiated in exactly one source file (qrw_qknorm_gc*.hip); the
// launcher (qrw_qknorm.hip) picks GC for the row and calls it.
//
// Definition: "TileLang tutorial, ch. 13", s2.4 (cross-module fusion: each
// q/k value gets a weighted RMSNorm and then RoPE; the q/k columns are read
// and written back and the v columns are not touched), with RMSNorm as in
// s3.2.1 taken over each head's head_dim channels and RoPE as in s3.3.1 on
// the head's tail span.
//
// Layout: a token row holds q_heads query heads, kv_heads key heads and
// kv_heads value heads of head_dim channels.  Only the first
// (q_heads + kv_heads) * head_dim channels are read and written.
//
// Mapping: the q/k part of a row is cut into chunks of 64*GC granules (GC
// chosen per row length so that the chunks split the row evenly, and one
// chunk covers the whole row when it has at most 768 granules); one wave64
// handles one chunk of one token, lane l taking granules
// chunk*64*GC + l + 64*g (g < GC), so every load and store instruction
// covers 1 KiB contiguous.  A head is HG = head_dim/8 consecutive lanes and
// chunks hold whole heads, so chunks are independent.  Per head: the sum of
// squares is reduced with DPP inside the head's HG lanes; the rotation pairs
// are in-lane (interleaved) or lane l and lane l ^ XR (NeoX, XR =
// rope_dim/16) inside the head's rotated span.  A lane's position in its
// head, hence its weight and table granule, is the same for all its granules.
//
// Arithmetic (binary32, one rounding at the output): u = x * w (exact for
// 16-bit operands), the rotation as one fma per output, then * rstd.
//
// With the KV-cache write (the same section's fusion table: Q/K RMSNorm +
// RoPE + quantised KV-cache write), the chunks cover the whole row: q heads
// are written back in place as above, while k heads (after norm and
// rotation) and v heads (as stored) are cast to E4M3FN with one scale per
// (token, head), the per-token cast of s3.1.5 applied to a head: scale =
// max(amax, 1e-4) / 448 from a DPP max inside the head's lanes, codes of the
// correctly rounded binary32 quotient, written to cache row slots[t].
#pragma once

#include <type_traits>

#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

// Destination of the quantised k and v heads (unused without the KV write).
struct KvDest {
  uint8_t* kc;             // [num_slots] rows of cache_stride bytes
  uint8_t* vc;
  float* ks;               // [num_slots, kv_heads]
  float* vs;
  const int64_t* slots;    // [tokens] or NULL (token t -> row t)
  int64_t num_slots;
  int64_t cache_stride;
  int k_end;               // first v granule of a row
  int kv_heads;
};

template <typename CS>
__device__ __forceinline__ const char* qk_table_row(const void* base, int64_t t, int half) {
  constexpr int bytes = std::is_same<CS, float>::value ? 4 : 2;
  return static_cast<const char*>(base) + t * (int64_t)half * bytes;
}

template <typename T, typename CS, bool NEOX, int HG, int XR, int GC, bool KV>
__global__ __launch_bounds__(kBlock) void qk_norm_rope_kernel(
    uint16_t* qkv, const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const void* cosv, const void* sinv, int64_t tokens, int64_t stride, int ng, int q_gran,
    int chunks, int s0, int half, float inv_n, float eps, KvDest kv) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t t = wave / chunks;
  if (t >= tokens) return;  // wave-uniform
  const int gb = (int)(wave - t * chunks) * kWave * GC;
  uint16_t* row = qkv + t * stride;
  const int j = lane & (HG - 1);        // granule position inside the head
  // NeoX with 2*XR == HG rotates the whole head (rope_dim == head_dim, s0 == 0):
  // every lane is in the span, known at compile time
  constexpr bool kWhole = NEOX && 2 * XR == HG;
  const int js = kWhole ? j : j - s0;   // position inside the rotated span (< 0: outside)
  const bool span = kWhole || js >= 0;
  int64_t slot = t;
  bool cached = true;
  if constexpr (KV) {
    if (kv.slots) slot = kv.slots[t];
    cached = slot >= 0 && slot < kv.num_slots;
  }

  u32x4 raw[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int gi = gb + kWave * g + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (gi < ng) raw[g] = ld16_stream(row + 8 * gi);
  }
  float fq[8], fk[8];
  if (wq) {
    widen8<T>(ld16(wq + 8 * j), fq);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) fq[e] = 1.0f;
  }
  if (wk) {
    widen8<T>(ld16(wk + 8 * j), fk);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) fk[e] = 1.0f;
  }
  float c[8], sn[8];
  const char* crow = qk_table_row<CS>(cosv, t, half);
  const char* srow = qk_table_row<CS>(sinv, t, half);
  if (NEOX) {
    const int tg = span ? (js & (XR - 1)) : 0;
    Table8<CS>::load(crow, tg, c);
    Table8<CS>::load(srow, tg, sn);
    if (js < XR) {  // first half of the span (or outside it): x c - x_partner s
#pragma unroll
      for (int e = 0; e < 8; ++e) sn[e] = -sn[e];
    }
  } else {
    float c4[4], s4[4];
    Table4<CS>::load(crow, span ? js : 0, c4);
    Table4<CS>::load(srow, span ? js : 0, s4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[k] = c4[k];
      sn[k] = s4[k];
    }
  }

  if constexpr (KV) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const int gi = gb + kWave * g + lane;
      const bool is_q = gi < q_gran;
      const bool is_v = KV && gi >= kv.k_end;
      float v[8];
      widen8<T>(raw[g], v);
      // q/k heads: weighted RMSNorm, then the rotation (value heads skip all of
      // it).  A head's lanes agree on is_q and is_v (the parts are whole heads),
      // so every group reduction below reads only lanes of its own head, and a
      // slot of value (query) heads skips the branches it does not need.
      auto norm_rotate = [&]() {
        float acc0 = 0.f, acc1 = 0.f;
        acc0 = sumsq2(T{}, raw[g][0], acc0);
        acc1 = sumsq2(T{}, raw[g][1], acc1);
        acc0 = sumsq2(T{}, raw[g][2], acc0);
        acc1 = sumsq2(T{}, raw[g][3], acc1);
        const float ss = group_sum<HG>(acc0 + acc1);
        // inv_n = 1 / head_dim, exact (head_dim is a power of two): ss * inv_n ==
        // ss / head_dim.  1/sqrt(mean + eps) once per head and granule (GC times
        // per lane): the hardware reciprocal square root refined by one
        // Newton-Raphson step, y <- y (3/2 - (v/2) y^2), good to about one
        // binary32 ulp.  A correctly rounded 1.0f / sqrtf() costs a division
        // sequence per head, which measured 7% slower on the 4096 x (32+8+8) x
        // 128 workload.
        const float mv = ss * inv_n + eps;
        float rstd = __builtin_amdgcn_rsqf(mv);
        rstd = rstd * fmaf(-0.5f * mv * rstd, rstd, 1.5f);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= is_q ? fq[e] : fk[e];
        if (NEOX) {
          float r[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = fmaf(v[e], c[e], lane_xor<XR>(v[e]) * sn[e]);
          if (span) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = r[e];
          }
        } else if (span) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float x0 = v[2 * k], x1 = v[2 * k + 1];
            v[2 * k] = fmaf(x0, c[k], -(x1 * sn[k]));
            v[2 * k + 1] = fmaf(x1, c[k], x0 * sn[k]);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= rstd;
      };
      if constexpr (KV) {
        if (!is_v) norm_rotate();
        if (is_q) {
          if (gi < ng) st16_stream(row + 8 * gi, narrow8<T>(v));
        } else {
          // k and v heads: one scale per (token, head) from the head's max
          float m = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
          const float am = fmaxf(group_max<HG>(m), 1e-4f);
          if (gi < ng && cached) {
            const float scale = scale_e4m3(am);
            const float y = recip_rn(scale);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], scale, y);
            const int hg = is_v ? gi - kv.k_end : gi - q_gran;  // granule inside the k (v) part
            st8_stream((is_v ? kv.vc : kv.kc) + slot * kv.cache_stride + 8 * hg, fp8x8(v));
            if (j == 0) (is_v ? kv.vs : kv.ks)[slot * kv.kv_heads + hg / HG] = scale;
          }
        }
      } else {
        norm_rotate();
        if (gi < ng) st16_stream(row + 8 * gi, narrow8<T>(v));
      }
    }
  } else {
    // in place: every granule of the chunk is a q or k granule
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const int gi = gb + kWave * g + lane;
      float acc0 = 0.f, acc1 = 0.f;
      acc0 = sumsq2(T{}, raw[g][0], acc0);
      acc1 = sumsq2(T{}, raw[g][1], acc1);
      acc0 = sumsq2(T{}, raw[g][2], acc0);
      acc1 = sumsq2(T{}, raw[g][3], acc1);
      const float ss = group_sum<HG>(acc0 + acc1);
      const bool is_q = gi < q_gran;
      // rstd as in the KV form's norm_rotate
      const float mv = ss * inv_n + eps;
      float rstd = __builtin_amdgcn_rsqf(mv);
      rstd = rstd * fmaf(-0.5f * mv * rstd, rstd, 1.5f);
      float v[8];
      widen8<T>(raw[g], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= is_q ? fq[e] : fk[e];
      if (NEOX) {
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = fmaf(v[e], c[e], lane_xor<XR>(v[e]) * sn[e]);
        if (span) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = r[e];
        }
      } else if (span) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = v[2 * k], x1 = v[2 * k + 1];
          v[2 * k] = fmaf(x0, c[k], -(x1 * sn[k]));
          v[2 * k + 1] = fmaf(x1, c[k], x0 * sn[k]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= rstd;
      if (gi < ng) st16_stream(row + 8 * gi, narrow8<T>(v));
    }
  }
}

// ------------------------------------------------------------------ dispatch
// Everything a launch needs besides the template arguments.
struct QkArgs {
  dim3 grid;
  hipStream_t st;
  uint16_t* x;
  const uint16_t* wq;
  const uint16_t* wk;
  const void* c;
  const void* s;
  int64_t tokens, stride;
  int ng, qg, chunks, s0, half;
  float inv_n, eps;
  KvDest kv;
  int dtype, cs_dtype, hg, xr;
  bool neox;
};

template <typename T, typename CS, bool NEOX, int HG, int XR, int GC>
void qk_go(const QkArgs& a) {
  if (a.kv.kc)
    qk_norm_rope_kernel<T, CS, NEOX, HG, XR, GC, true><<<a.grid, kBlock, 0, a.st>>>(
        a.x, a.wq, a.wk, a.c, a.s, a.tokens, a.stride, a.ng, a.qg, a.chunks, a.s0, a.half,
        a.inv_n, a.eps, a.kv);
  else
    qk_norm_rope_kernel<T, CS, NEOX, HG, XR, GC, false><<<a.grid, kBlock, 0, a.st>>>(
        a.x, a.wq, a.wk, a.c, a.s, a.tokens, a.stride, a.ng, a.qg, a.chunks, a.s0, a.half,
        a.inv_n, a.eps, a.kv);
}

template <typename T, typename CS, bool NEOX, int HG, int GC>
void qk_go_xr(const QkArgs& a) {
  if constexpr (!NEOX) {
    qk_go<T, CS, NEOX, HG, 1, GC>(a);
  } else {
    switch (a.xr) {
      case 1: qk_go<T, CS, NEOX, HG, 1, GC>(a); break;
      case 2: qk_go<T, CS, NEOX, HG, 2, GC>(a); break;
      case 4: qk_go<T, CS, NEOX, HG, 4, GC>(a); break;
      case 8:  // rope_dim <= head_dim keeps xr <= hg / 2
        if constexpr (HG >= 16) qk_go<T, CS, NEOX, HG, 8, GC>(a);
        break;
      default:
        if constexpr (HG >= 32) qk_go<T, CS, NEOX, HG, 16, GC>(a);
        break;
    }
  }
}

template <typename T, typename CS, bool NEOX, int GC>
void qk_go_hg(const QkArgs& a) {
  switch (a.hg) {
    case 8: qk_go_xr<T, CS, NEOX, 8, GC>(a); break;
    case 16: qk_go_xr<T, CS, NEOX, 16, GC>(a); break;
    default: qk_go_xr<T, CS, NEOX, 32, GC>(a); break;
  }
}

// All kernels of chunk width GC: dtype, table dtype and pairing dispatched at
// run time.
template <int GC>
void qk_run(const QkArgs& a) {
  if (a.dtype == 1) {
    if (a.cs_dtype == 3) {
      if (a.neox) qk_go_hg<F16, float, true, GC>(a);
      else qk_go_hg<F16, float, false, GC>(a);
    } else {
      if (a.neox) qk_go_hg<F16, F16, true, GC>(a);
      else qk_go_hg<F16, F16, false, GC>(a);
    }
  } else {
    if (a.cs_dtype == 3) {
      if (a.neox) qk_go_hg<BF16, float, true, GC>(a);
      else qk_go_hg<BF16, float, false, GC>(a);
    } else {
      if (a.neox) qk_go_hg<BF16, BF16, true, GC>(a);
      else qk_go_hg<BF16, BF16, false, GC>(a);
    }
  }
}

// One entry per chunk width, each defined (and its kernels instantiated) in a
// single source file.
void qk_run_gc1(const QkArgs& a);
void qk_run_gc2(const QkArgs& a);
void qk_run_gc3(const QkArgs& a);
void qk_run_gc4(const QkArgs& a);
void qk_run_gc5(const QkArgs& a);
void qk_run_gc6(const QkArgs& a);
void qk_run_gc8(const QkArgs& a);
void qk_run_gc10(const QkArgs& a);
void qk_run_gc12(const QkArgs& a);

}  // namespace qrw
