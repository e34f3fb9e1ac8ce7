// qrw_contig.h -- index math of the contiguous lane mapping shared by the
// RoPE kernel (qrw_rope_contig.hip) and the fused operator's tail-rotation
// kernel (qrw_fused_tail.hip).  Plain C++ usable on host and device, so the
// CPU test suite checks it over every accepted shape before any launch.
//
// Mapping: a token row of heads * head_dim channels is 64 * G granules of 8
// channels; lane l of the token's wave owns granules l + 64 g, g < G, so each
// load and store instruction covers one contiguous block.  A head is
// HG = head_dim / 8 granules (a power of two); its last rope_dim / 8 granules
// rotate ("TileLang tutorial, ch. 13", s3.3.1: the tail span of each head),
// from position s0 = HG - rope_dim / 8 on.  With rope_dim <= 256 the span is
// at most 32 granules, so:
//   * a head of at most 64 granules sits at the same lanes in every step, and
//     a longer head rotates in one step of its own, at lanes s0 mod 64 and up:
//     a lane's position in the span (hence its table granule) is the same in
//     every step that rotates it;
//   * the NeoX partner of span position j is j ^ (rope_dim / 16), which is
//     lane l ^ (rope_dim / 16) of the same step (the span starts at a multiple
//     of rope_dim / 8, and rope_dim / 16 < 64);
//   * interleaved pairs (channels 2k, 2k + 1) sit inside one granule.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define QRW_CHD __host__ __device__ __forceinline__
#else
#define QRW_CHD inline
#endif

namespace qrw {

// Position of lane l's granules in the rotated span, in the steps that
// rotate them (negative: the lane never rotates).  hg_mask = HG - 1.
QRW_CHD int contig_span_pos(int lane, int hg_mask, int s0) {
  return (lane & hg_mask & 63) - (s0 & 63);
}

// Whether granule gi of the row rotates.
QRW_CHD bool contig_rotates(int gi, int hg_mask, int s0) { return (gi & hg_mask) >= s0; }

// Granule blocks per lane (G) for the contiguous RoPE path, or 0 when it does
// not apply: head_dim and rope_dim powers of two with 16 <= rope_dim <=
// min(head_dim, 256), and a row of 512 * G channels, G in {1, 2, 4, 8, 16};
// or G in {3, 5, 6, 7, 10, 12, 14} for heads of 64 or 128, interleaved, or
// NeoX rotating whole heads.
QRW_CHD int rope_contig_blocks(int64_t heads, int64_t head_dim, int64_t rope_dim, bool neox) {
  const bool p2 = head_dim > 0 && (head_dim & (head_dim - 1)) == 0 && rope_dim > 0 &&
                  (rope_dim & (rope_dim - 1)) == 0;
  if (!p2 || rope_dim < 16 || rope_dim > head_dim || rope_dim > 256 || heads < 1) return 0;
  const int64_t n = heads * head_dim;
  if (n % 512 != 0) return 0;
  const int64_t g = n / 512;
  if (g == 1 || g == 2 || g == 4 || g == 8 || g == 16) return (int)g;
  const bool odd_ok = (head_dim == 64 || head_dim == 128) && (!neox || rope_dim == head_dim);
  const bool odd_g = g == 3 || g == 5 || g == 6 || g == 7 || g == 10 || g == 12 || g == 14;
  return odd_ok && odd_g ? (int)g : 0;
}

}  // namespace qrw
