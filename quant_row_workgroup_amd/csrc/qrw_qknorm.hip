// qrw_qknorm.hip -- per-head QK RMSNorm + RoPE, in place on a packed QKV row
// (gfx950).
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
// Mapping: the q/k part of a row is cut into chunks of 64*GC granules; one
// wave64 handles one chunk of one token, lane l taking granules
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
#include <type_traits>

#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

// Sum over aligned groups of L consecutive lanes (L = 8, 16 or 32); every
// lane of a group receives the same value.
template <int L>
__device__ __forceinline__ float head_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp<kDppMirror>(v);
  if constexpr (L >= 32) v += lane_xor<16>(v);
  return v;
}

template <typename CS>
__device__ __forceinline__ const char* qk_table_row(const void* base, int64_t t, int half) {
  constexpr int bytes = std::is_same<CS, float>::value ? 4 : 2;
  return static_cast<const char*>(base) + t * (int64_t)half * bytes;
}

template <typename T, typename CS, bool NEOX, int HG, int XR, int GC>
__global__ __launch_bounds__(kBlock) void qk_norm_rope_kernel(
    uint16_t* qkv, const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const void* cosv, const void* sinv, int64_t tokens, int64_t stride, int ng, int q_gran,
    int chunks, int s0, int half, float n_f, float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t t = wave / chunks;
  if (t >= tokens) return;  // wave-uniform
  const int gb = (int)(wave - t * chunks) * kWave * GC;
  uint16_t* row = qkv + t * stride;
  const int j = lane & (HG - 1);        // granule position inside the head
  const int js = j - s0;                // position inside the rotated span (< 0: outside)
  const bool span = js >= 0;

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

#pragma unroll
  for (int g = 0; g < GC; ++g) {
    const int gi = gb + kWave * g + lane;
    float acc0 = 0.f, acc1 = 0.f;
    acc0 = sumsq2(T{}, raw[g][0], acc0);
    acc1 = sumsq2(T{}, raw[g][1], acc1);
    acc0 = sumsq2(T{}, raw[g][2], acc0);
    acc1 = sumsq2(T{}, raw[g][3], acc1);
    const float ss = head_sum<HG>(acc0 + acc1);
    const float rstd = 1.0f / sqrtf(ss / n_f + eps);
    float v[8];
    widen8<T>(raw[g], v);
    const bool is_q = gi < q_gran;
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

// ------------------------------------------------------------------ launch
namespace {

constexpr int kQkChunk = 2;  // granules per lane per wave

template <typename T, typename CS, bool NEOX, int HG, int XR>
void qk_go(dim3 grid, hipStream_t st, uint16_t* x, const uint16_t* wq, const uint16_t* wk,
           const void* c, const void* s, int64_t tokens, int64_t stride, int ng, int qg,
           int chunks, int s0, int half, float n_f, float eps) {
  qk_norm_rope_kernel<T, CS, NEOX, HG, XR, kQkChunk><<<grid, kBlock, 0, st>>>(
      x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
}

template <typename T, typename CS, bool NEOX, int HG>
void qk_go_xr(int xr, dim3 grid, hipStream_t st, uint16_t* x, const uint16_t* wq,
              const uint16_t* wk, const void* c, const void* s, int64_t tokens, int64_t stride,
              int ng, int qg, int chunks, int s0, int half, float n_f, float eps) {
  if constexpr (!NEOX) {
    qk_go<T, CS, NEOX, HG, 1>(grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
  } else {
    switch (xr) {
      case 1: qk_go<T, CS, NEOX, HG, 1>(grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps); break;
      case 2: qk_go<T, CS, NEOX, HG, 2>(grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps); break;
      case 4: qk_go<T, CS, NEOX, HG, 4>(grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps); break;
      case 8:  // rope_dim <= head_dim keeps xr <= hg / 2
        if constexpr (HG >= 16) qk_go<T, CS, NEOX, HG, 8>(grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
        break;
      default:
        if constexpr (HG >= 32) qk_go<T, CS, NEOX, HG, 16>(grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
        break;
    }
  }
}

template <typename T, typename CS, bool NEOX>
void qk_go_hg(int hg, int xr, dim3 grid, hipStream_t st, uint16_t* x, const uint16_t* wq,
              const uint16_t* wk, const void* c, const void* s, int64_t tokens, int64_t stride,
              int ng, int qg, int chunks, int s0, int half, float n_f, float eps) {
  switch (hg) {
    case 8: qk_go_xr<T, CS, NEOX, 8>(xr, grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps); break;
    case 16: qk_go_xr<T, CS, NEOX, 16>(xr, grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps); break;
    default: qk_go_xr<T, CS, NEOX, 32>(xr, grid, st, x, wq, wk, c, s, tokens, stride, ng, qg, chunks, s0, half, n_f, eps); break;
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(void* qkv, const void* q_weight, const void* k_weight,
                               const void* cos, const void* sin, int64_t tokens, int64_t q_heads,
                               int64_t kv_heads, int64_t head_dim, int64_t rope_dim,
                               int64_t stride, int dtype, int cs_dtype, bool neox, float eps,
                               hipStream_t stream) {
  const int hg = (int)(head_dim / 8);
  const int xr = (int)(rope_dim / 16);
  const int ng = (int)((q_heads + kv_heads) * hg);
  const int qg = (int)(q_heads * hg);
  const int per_wave = kWave * kQkChunk;
  const int chunks = (ng + per_wave - 1) / per_wave;
  const int s0 = (int)((head_dim - rope_dim) / 8);
  const int half = (int)(rope_dim / 2);
  const int64_t waves = tokens * chunks;
  const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
  auto* x = static_cast<uint16_t*>(qkv);
  const auto* wq = static_cast<const uint16_t*>(q_weight);
  const auto* wk = static_cast<const uint16_t*>(k_weight);
  const float n_f = (float)head_dim;
  if (dtype == 1) {
    if (cs_dtype == 3) {
      if (neox) qk_go_hg<F16, float, true>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
      else qk_go_hg<F16, float, false>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
    } else {
      if (neox) qk_go_hg<F16, F16, true>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
      else qk_go_hg<F16, F16, false>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
    }
  } else {
    if (cs_dtype == 3) {
      if (neox) qk_go_hg<BF16, float, true>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
      else qk_go_hg<BF16, float, false>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
    } else {
      if (neox) qk_go_hg<BF16, BF16, true>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
      else qk_go_hg<BF16, BF16, false>(hg, xr, grid, stream, x, wq, wk, cos, sin, tokens, stride, ng, qg, chunks, s0, half, n_f, eps);
    }
  }
  return hipGetLastError();
}

}  // namespace qrw
