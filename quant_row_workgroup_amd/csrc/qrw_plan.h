// qrw_plan.h -- how one token row of the RoPE and fused kernels is split
// into lane work items.  Plain C++ usable on host and device, so the CPU test
// suite can check bounds and coverage of every offset before any launch.
//
// A token row holds `heads` heads of `head_dim` channels.  In each head the
// tail span of `rope_dim` channels rotates; the first P = head_dim - rope_dim
// channels pass through (the partial rotation of "TileLang tutorial, ch. 13",
// s3.3.1).  The row is cut into 16-byte granules of 8 channels and the
// granules are grouped into items of two:
//   * rope item (h, s), s in [0, rope_dim/16):
//       NeoX half-split  A = span + 8s,   B = A + rope_dim/2
//       interleaved      A = span + 16s,  B = A + 8
//     so every rotation pair lies inside one item (NeoX pairs channel e of A
//     with channel e of B; interleaved pairs sit inside A or inside B), and
//     both conventions use table entries [8s, 8s+8) of the token's cos/sin row.
//   * plain item j: pass-through granules 2j and 2j+1 of the row's plain
//     granules in row order (B absent when their count is odd).
// Rope items come first, then plain items.  Lane l of a wave takes items
// l, l+64, l+128, ...; with pairs lane-local, no cross-lane exchange is needed.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define QRW_HD __host__ __device__ __forceinline__
#else
#define QRW_HD inline
#endif

namespace qrw {

// Unsigned division of n < 2^16 by a fixed d in [1, 2^16) with one multiply:
// floor(n / d) == (n * ceil(2^32 / d)) >> 32 because n * (ceil(2^32/d)*d - 2^32)
// < n * d < 2^32.
struct FastDiv {
  uint64_t magic;
  int d;
};

inline FastDiv make_fastdiv(int d) {
  FastDiv f;
  f.d = d < 1 ? 1 : d;
  f.magic = ((uint64_t(1) << 32) + uint64_t(f.d) - 1) / uint64_t(f.d);
  return f;
}

QRW_HD int fastdiv(const FastDiv& f, int n) {
  return (int)((uint64_t(uint32_t(n)) * f.magic) >> 32);
}

enum ItemKind { kItemNone = 0, kItemRope = 1, kItemPlain = 2 };

struct RowPlan {
  int head_dim;
  int rope_dim;
  int pass;      // pass-through channels per head (head_dim - rope_dim)
  int half;      // rope_dim / 2
  int gph;       // rope items per head (rope_dim / 16)
  int gpp;       // plain granules per head (pass / 8)
  int n_rope;    // rope items per token
  int n_plain;   // plain granules per token
  int n_items;   // all items per token
  int n;         // channels per token (heads * head_dim)
  int lane_hoist;  // 1 if every rope item of lane l uses table granule l % gph
  FastDiv div_gph;
  FastDiv div_gpp;
};

inline RowPlan make_plan(int64_t heads, int64_t head_dim, int64_t rope_dim) {
  RowPlan p;
  p.head_dim = (int)head_dim;
  p.rope_dim = (int)rope_dim;
  p.pass = (int)(head_dim - rope_dim);
  p.half = (int)(rope_dim / 2);
  p.gph = (int)(rope_dim / 16);
  p.gpp = p.pass / 8;
  p.n_rope = (int)heads * p.gph;
  p.n_plain = (int)heads * p.gpp;
  p.n_items = p.n_rope + (p.n_plain + 1) / 2;
  p.n = (int)(heads * head_dim);
  p.lane_hoist = (64 % p.gph) == 0 ? 1 : 0;
  p.div_gph = make_fastdiv(p.gph);
  p.div_gpp = make_fastdiv(p.gpp);
  return p;
}

// Element offset (within the token row) of plain granule j.
QRW_HD int plain_offset(const RowPlan& p, int j) {
  const int h = fastdiv(p.div_gpp, j);
  return h * p.head_dim + 8 * (j - h * p.gpp);
}

// Offsets of item `it`: A and B (B = -1 when absent) and the table granule s.
QRW_HD int item_offsets(const RowPlan& p, int it, bool neox, int& a, int& b, int& s) {
  a = -1;
  b = -1;
  s = 0;
  if (it < p.n_rope) {
    const int h = fastdiv(p.div_gph, it);
    s = it - h * p.gph;
    const int span = h * p.head_dim + p.pass;
    a = neox ? span + 8 * s : span + 16 * s;
    b = neox ? a + p.half : a + 8;
    return kItemRope;
  }
  const int j = 2 * (it - p.n_rope);
  if (j >= p.n_plain) return kItemNone;
  a = plain_offset(p, j);
  if (j + 1 < p.n_plain) b = plain_offset(p, j + 1);
  return kItemPlain;
}

}  // namespace qrw
