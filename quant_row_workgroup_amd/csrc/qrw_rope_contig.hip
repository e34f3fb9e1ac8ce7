// qrw_rope_contig.hip -- RoPE, interleaved and NeoX half-split, in the
// contiguous lane mapping (gfx950).
//
// Definition: "TileLang tutorial, ch. 13", s3.3.1 (the two pairings, the
// cos/sin table of shape (positions, rope_dim / 2), rotation of each head's
// tail span) and s3.3.2 (binary32 math, one final cast).
//
// Mapping (qrw_contig.h): one wave64 per token, four tokens per workgroup;
// lane l owns granules l, l + 64, ..., so every load and store instruction
// covers 1 KiB of the row.  A lane reads its one table granule up front,
// beside its row.  Interleaved pairs sit inside a granule; a NeoX pair's
// partner is lane l ^ (rope_dim / 16) of the same step, read with a lane
// exchange.  Granules outside the rotated span are stored as loaded (or not
// at all in place).  Arithmetic as the item kernel's rotate(): first of a
// pair x_a c - x_b s as fma(x_a, c, -(x_b s)), second fma(x_b, c, x_a s), so
// both kernels give the same bits.
//
// Measured on MI355X against the item kernel (qrw_rope.hip), 4096 tokens,
// outputs identical: 32 heads x 128 f16 with binary32 tables 11.48 against
// 20.70 us interleaved and 11.87 against 12.45 us NeoX; rotating 64 of 128
// channels 11.92 against 21.32 us interleaved and 12.18 against 17.47 us
// NeoX.  Eight rows per workgroup measured slower than four.
#include "qrw_contig.h"
#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

template <typename T, typename CS, bool NEOX, int G, int XR>
__global__ __launch_bounds__(kBlock) void rope_contig_kernel(const uint16_t* x, const void* cosv,
                                                             const void* sinv, uint16_t* y,
                                                             int64_t tokens, int64_t xs,
                                                             int64_t ys, int half, int hg_mask,
                                                             int s0, int copy) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= tokens) return;  // wave-uniform
  const uint16_t* xr = x + t * xs;
  uint16_t* yr = y + t * ys;
  u32x4 r[G];
#pragma unroll
  for (int g = 0; g < G; ++g) r[g] = ld16_stream(xr + 8 * (kWave * g + lane));
  const int jl = contig_span_pos(lane, hg_mask, s0);
  const char* crow = table_row<CS>(cosv, t, half);
  const char* srow = table_row<CS>(sinv, t, half);
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
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int gi = kWave * g + lane;
    const bool span = contig_rotates(gi, hg_mask, s0);
    uint16_t* p = yr + 8 * gi;
    if (__builtin_amdgcn_ballot_w64(span) != 0) {  // wave-uniform: some lane rotates
      float v[8];
      widen8<T>(r[g], v);
      if (NEOX) {
        // every lane takes part in the exchange; lanes outside the span keep x
        float rv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rv[e] = fmaf(v[e], c[e], lane_xor<XR>(v[e]) * sn[e]);
        if (span) st16_stream(p, narrow8<T>(rv));
        else if (copy) st16_stream(p, r[g]);
      } else if (span) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = v[2 * k], x1 = v[2 * k + 1];
          v[2 * k] = fmaf(x0, c[k], -(x1 * sn[k]));
          v[2 * k + 1] = fmaf(x1, c[k], x0 * sn[k]);
        }
        st16_stream(p, narrow8<T>(v));
      } else if (copy) {
        st16_stream(p, r[g]);
      }
    } else if (copy) {
      st16_stream(p, r[g]);
    }
  }
}

namespace {

struct RopeArgs {
  dim3 grid;
  hipStream_t st;
  const uint16_t* x;
  const void* c;
  const void* s;
  uint16_t* y;
  int64_t tokens, xs, ys;
  int half, hg_mask, s0, copy;
};

template <typename T, typename CS, bool NEOX, int G, int XR>
void rc_launch(const RopeArgs& a) {
  rope_contig_kernel<T, CS, NEOX, G, XR><<<a.grid, kBlock, 0, a.st>>>(
      a.x, a.c, a.s, a.y, a.tokens, a.xs, a.ys, a.half, a.hg_mask, a.s0, a.copy);
}

template <typename T, typename CS, bool NEOX, int G>
void rc_xr(int xr, const RopeArgs& a) {
  if constexpr (!NEOX) {
    rc_launch<T, CS, NEOX, G, 1>(a);
  } else {
    switch (xr) {
      case 1: rc_launch<T, CS, NEOX, G, 1>(a); break;
      case 2: rc_launch<T, CS, NEOX, G, 2>(a); break;
      case 4: rc_launch<T, CS, NEOX, G, 4>(a); break;
      case 8: rc_launch<T, CS, NEOX, G, 8>(a); break;
      default: rc_launch<T, CS, NEOX, G, 16>(a); break;
    }
  }
}

// The other block counts: heads of 64 or 128 (NeoX: whole heads, rope_dim / 16
// = 4 or 8), which keeps the instance count down.
template <typename T, typename CS, bool NEOX, int G>
void rc_xr48(int xr, const RopeArgs& a) {
  if constexpr (!NEOX) {
    rc_launch<T, CS, NEOX, G, 1>(a);
  } else {
    if (xr == 4) rc_launch<T, CS, NEOX, G, 4>(a);
    else rc_launch<T, CS, NEOX, G, 8>(a);
  }
}

template <typename T, typename CS, bool NEOX>
void rc_g(int g, int xr, const RopeArgs& a) {
  switch (g) {
    case 1: rc_xr<T, CS, NEOX, 1>(xr, a); break;
    case 2: rc_xr<T, CS, NEOX, 2>(xr, a); break;
    case 3: rc_xr48<T, CS, NEOX, 3>(xr, a); break;
    case 4: rc_xr<T, CS, NEOX, 4>(xr, a); break;
    case 5: rc_xr48<T, CS, NEOX, 5>(xr, a); break;
    case 6: rc_xr48<T, CS, NEOX, 6>(xr, a); break;
    case 7: rc_xr48<T, CS, NEOX, 7>(xr, a); break;
    case 8: rc_xr<T, CS, NEOX, 8>(xr, a); break;
    case 10: rc_xr48<T, CS, NEOX, 10>(xr, a); break;
    case 12: rc_xr48<T, CS, NEOX, 12>(xr, a); break;
    case 14: rc_xr48<T, CS, NEOX, 14>(xr, a); break;
    default: rc_xr<T, CS, NEOX, 16>(xr, a); break;
  }
}

template <typename T, typename CS>
void rc_neox(bool neox, int g, int xr, const RopeArgs& a) {
  if (neox) rc_g<T, CS, true>(g, xr, a);
  else rc_g<T, CS, false>(g, xr, a);
}

}  // namespace

bool rope_contig_ok(int64_t heads, int64_t head_dim, int64_t rope_dim, bool neox) {
  return rope_contig_blocks(heads, head_dim, rope_dim, neox) != 0;
}

hipError_t launch_rope_contig(const void* x, const void* cos, const void* sin, void* y,
                              int64_t tokens, int64_t heads, int64_t head_dim, int64_t rope_dim,
                              int64_t xs, int64_t ys, int dtype, int cs_dtype, bool neox,
                              hipStream_t stream) {
  const int g = rope_contig_blocks(heads, head_dim, rope_dim, neox);
  if (g == 0) return hipErrorInvalidValue;  // callers check rope_contig_ok first
  RopeArgs a;
  a.grid = dim3((unsigned)((tokens + kRowsPerBlock - 1) / kRowsPerBlock));
  a.st = stream;
  a.x = static_cast<const uint16_t*>(x);
  a.c = cos;
  a.s = sin;
  a.y = static_cast<uint16_t*>(y);
  a.tokens = tokens;
  a.xs = xs;
  a.ys = ys;
  a.half = (int)(rope_dim / 2);
  a.hg_mask = (int)(head_dim / 8 - 1);
  a.s0 = (int)((head_dim - rope_dim) / 8);
  a.copy = (x != y) ? 1 : 0;  // in place: pass-through channels are already there
  const int xr = (int)(rope_dim / 16);
  if (dtype == 1) {
    if (cs_dtype == 3) rc_neox<F16, float>(neox, g, xr, a);
    else rc_neox<F16, F16>(neox, g, xr, a);
  } else {
    if (cs_dtype == 3) rc_neox<BF16, float>(neox, g, xr, a);
    else rc_neox<BF16, BF16>(neox, g, xr, a);
  }
  return hipGetLastError();
}

}  // namespace qrw
