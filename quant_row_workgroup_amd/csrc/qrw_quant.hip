// qrw_quant.hip -- activation quantisation to OCP E4M3FN, one scale per token
// or per group of consecutive channels (gfx950).
//
// Definition: "TileLang tutorial, ch. 13", s3.1.5 (the per-token / per-group
// cast): amax over the group -> scale = max(amax, 1e-4) / fp8_max -> codes of
// clamp(x / scale, -fp8_max, fp8_max), fp8_max = 448 for E4M3FN.
//
// Mapping: one wave64 per row; lane l owns granules l, l+64, ... (GPL of
// them), so each load instruction covers 1 KiB of contiguous row and each
// code store 512 B.  A group of `group` channels is group/8 consecutive lanes
// of one load instruction; its amax is reduced with DPP inside the lane group
// (quad permutes, half-row and row mirrors) or with the LDS crossbar for 32
// lanes, and for a whole-row group with the wave reduction.  x is read and the
// codes are written with non-temporal hints (measured faster on MI355X).
//
// The code of x is the E4M3 rounding of the binary32 quotient x / scale, as
// the page's cast computes it in float32.  The quotient is formed correctly
// rounded without a division per element (Markstein's correction): with
// y = RN(1/scale) once per group, q = RN(x*y), r = x - q*scale (exact, one
// fma), RN(q + r*y) is RN(x/scale).  |x| <= amax makes the largest quotient
// at most 448 * (1 + 2^-23) < 464, so the conversion stays finite and the
// clamp cannot act.
#include "qrw_device.h"
#include "qrw_launch.h"

namespace qrw {

// SEG: rows longer than one wave holds (QRW_MAX_ROW) are cut into segments of
// GPL * 64 granules (4096 or 2048 channels; with FULL every segment is whole,
// else the last one is shorter), one wave per (row, segment); groups never
// straddle a segment.  Otherwise a wave takes a whole row.

template <typename T, int GPL, bool FULL, int L, bool SEG>
__global__ __launch_bounds__(kBlock) void act_quant_group_kernel(const uint16_t* x, uint8_t* q,
                                                                 float* scales, int64_t rows,
                                                                 int ng, int64_t xs, int64_t qs,
                                                                 int64_t groups, int segs) {
  // When a whole row (segment) has at most 64 groups (GPL <= L), lane j
  // collects the scale of group j (from any lane of that group, by a lane
  // permute) and the scales leave in one contiguous store instead of one
  // store per group.
  constexpr bool kGather = FULL && GPL <= L;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t row = SEG ? wave / segs : wave;
  if (row >= rows) return;  // wave-uniform
  const int seg = SEG ? (int)(wave - row * segs) : 0;
  const int g0 = seg * GPL * kWave;  // first granule of the segment
  const uint16_t* xr = x + row * xs + 8 * (int64_t)g0;
  uint8_t* qr = q + row * qs + 8 * (int64_t)g0;
  float* sr = scales + row * groups + g0 / L;
  if (SEG) ng = min(ng - g0, GPL * kWave);  // granules in this segment
  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16_stream(xr + 8 * gi);
  }
  float mine = 0.0f;
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    float v[8];
    widen8<T>(raw[g], v);
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) m = fmaxf(m, fmaxf(fabsf(v[e]), fabsf(v[e + 1])));
    const float am = fmaxf(group_max<L>(m), 1e-4f);  // groups never straddle the row end
    const float scale = scale_e4m3(am);
    if constexpr (kGather) {
      // groups g*(64/L) .. of this step sit in lane blocks of L; lane j takes
      // group j = g*(64/L) + q from lane q*L
      constexpr int kPer = kWave / L;
      const int src = (lane % kPer) * L;
      const float got = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(src * 4, __builtin_bit_cast(int, scale)));
      if (lane / kPer == g) mine = got;
    }
    if (FULL || gi < ng) {
      const float y = recip_rn(scale);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], scale, y);
      st8_stream(qr + 8 * gi, fp8x8(v));
      if (!kGather && (lane & (L - 1)) == 0) sr[gi / L] = scale;
    }
  }
  if constexpr (kGather) {
    if (lane < GPL * (kWave / L)) sr[lane] = mine;
  }
}

// One scale per row.
template <typename T, int GPL, bool FULL>
__global__ __launch_bounds__(kBlock) void act_quant_token_kernel(const uint16_t* x, uint8_t* q,
                                                                 float* scales, int64_t rows,
                                                                 int ng, int64_t xs,
                                                                 int64_t qs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * xs;
  uint8_t* qr = q + row * qs;
  u32x4 raw[GPL];
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16_stream(xr + 8 * gi);
  }
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      m[e >> 1] = fmaxf(m[e >> 1], fmaxf(fabsf(v[e]), fabsf(v[e + 1])));
  }
  const float am = fmaxf(wave_max(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]))), 1e-4f);
  const float scale = scale_e4m3(am);
  const float y = recip_rn(scale);
  if (lane == 0) scales[row] = scale;
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int gi = g * kWave + lane;
    if (FULL || gi < ng) {
      float v[8];
      widen8<T>(raw[g], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], scale, y);
      st8_stream(qr + 8 * gi, fp8x8(v));
    }
  }
}

// One scale per row for rows longer than one wave holds: one workgroup of
// kQuantBlockWaves waves per row, thread t owning granules t, t + 1024, ...
// (GPT of them).  The row's amax is the maximum of the wave maxima, gathered
// through LDS behind one barrier (a maximum is exact in any order, so the
// scale is the one the one-wave kernel would form), then the same quotient.
constexpr int kQuantBlockWaves = 16;

template <typename T, int GPT, bool FULL>
__global__ __launch_bounds__(kWave * kQuantBlockWaves) void act_quant_token_block_kernel(
    const uint16_t* x, uint8_t* q, float* scales, int ng, int64_t xs, int64_t qs) {
  constexpr int HT = kWave * kQuantBlockWaves;
  __shared__ float slot[kQuantBlockWaves];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * xs;
  uint8_t* qr = q + row * qs;
  u32x4 raw[GPT];
#pragma unroll
  for (int g = 0; g < GPT; ++g) {
    const int gi = g * HT + t;
    raw[g] = (u32x4){0u, 0u, 0u, 0u};
    if (FULL || gi < ng) raw[g] = ld16_stream(xr + 8 * gi);
  }
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < GPT; ++g) {
    float v[8];
    widen8<T>(raw[g], v);
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      m[e >> 1] = fmaxf(m[e >> 1], fmaxf(fabsf(v[e]), fabsf(v[e + 1])));
  }
  const float wm = wave_max(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])));
  if ((t & (kWave - 1)) == 0) slot[t >> 6] = wm;
  __syncthreads();
  float am = slot[0];
#pragma unroll
  for (int i = 1; i < kQuantBlockWaves; ++i) am = fmaxf(am, slot[i]);
  const float scale = scale_e4m3(fmaxf(am, 1e-4f));
  const float y = recip_rn(scale);
  if (t == 0) scales[row] = scale;
#pragma unroll
  for (int g = 0; g < GPT; ++g) {
    const int gi = g * HT + t;
    if (FULL || gi < ng) {
      float v[8];
      widen8<T>(raw[g], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], scale, y);
      st8_stream(qr + 8 * gi, fp8x8(v));
    }
  }
}

// ------------------------------------------------------------------ launch
namespace {

int quant_gpl(int ng) { return ng <= 64 ? 1 : ng <= 128 ? 2 : ng <= 256 ? 4 : ng <= 512 ? 8 : 16; }

template <typename T, int GPL, bool FULL, bool SEG = false>
void group_go(int lanes, dim3 grid, hipStream_t st, const uint16_t* x, uint8_t* q, float* sc,
              int64_t rows, int ng, int64_t xs, int64_t qs, int64_t groups, int segs = 1) {
  switch (lanes) {
    case 1: act_quant_group_kernel<T, GPL, FULL, 1, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
    case 2: act_quant_group_kernel<T, GPL, FULL, 2, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
    case 4: act_quant_group_kernel<T, GPL, FULL, 4, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
    case 8: act_quant_group_kernel<T, GPL, FULL, 8, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
    case 16: act_quant_group_kernel<T, GPL, FULL, 16, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
    case 32: act_quant_group_kernel<T, GPL, FULL, 32, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
    default: act_quant_group_kernel<T, GPL, FULL, 64, SEG><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs, groups, segs); break;
  }
}

template <typename T, int GPL, bool FULL>
void quant_go(int64_t group, int64_t n, dim3 grid, hipStream_t st, const uint16_t* x, uint8_t* q,
              float* sc, int64_t rows, int ng, int64_t xs, int64_t qs) {
  if (group == n)
    act_quant_token_kernel<T, GPL, FULL><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs);
  else
    group_go<T, GPL, FULL>((int)(group / 8), grid, st, x, q, sc, rows, ng, xs, qs, n / group);
}

// Rows longer than one wave holds: per group, waves on 4096-channel segments;
// per token, one workgroup per row.
template <typename T>
void quant_long(int64_t group, int64_t n, hipStream_t st, const uint16_t* x, uint8_t* q,
                float* sc, int64_t rows, int64_t xs, int64_t qs) {
  const int ng = (int)(n / 8);
  if (group == n) {
    const int gpt = (ng + kWave * kQuantBlockWaves - 1) / (kWave * kQuantBlockWaves);
    const int g = gpt <= 2 ? 2 : gpt <= 4 ? 4 : 8;  // ng <= 8192: at most 8
    const bool full = ng == g * kWave * kQuantBlockWaves;
    const dim3 grid((unsigned)rows);
    const dim3 block(kWave * kQuantBlockWaves);
#define QRW_AQ_BLOCK(G)                                                                         \
  if (full) act_quant_token_block_kernel<T, G, true><<<grid, block, 0, st>>>(x, q, sc, ng, xs, qs); \
  else act_quant_token_block_kernel<T, G, false><<<grid, block, 0, st>>>(x, q, sc, ng, xs, qs);
    if (g == 2) { QRW_AQ_BLOCK(2) }
    else if (g == 4) { QRW_AQ_BLOCK(4) }
    else { QRW_AQ_BLOCK(8) }
#undef QRW_AQ_BLOCK
    return;
  }
  // whole segments of 512 granules, else of 256 (e.g. rows of 14336 or 18432
  // channels), else 512 with a shorter last one
  const int gpl = ng % 512 == 0 ? 8 : ng % 256 == 0 ? 4 : 8;
  const bool full = ng % (gpl * kWave) == 0;
  const int segs = (ng + gpl * kWave - 1) / (gpl * kWave);
  const int64_t waves = rows * segs;
  const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
  const int lanes = (int)(group / 8);
  if (gpl == 4)
    group_go<T, 4, true, true>(lanes, grid, st, x, q, sc, rows, ng, xs, qs, n / group, segs);
  else if (full)
    group_go<T, 8, true, true>(lanes, grid, st, x, q, sc, rows, ng, xs, qs, n / group, segs);
  else
    group_go<T, 8, false, true>(lanes, grid, st, x, q, sc, rows, ng, xs, qs, n / group, segs);
}

// Whole rows of 64 * e granules, e not a power of two (hidden sizes 1536 ...
// 7168): per token, one-wave instances of their own (e = 3, 5, 6, 7, 10, 12,
// 14); per group, when the row splits into segments of 128, 256 or 512
// granules, waves on those segments.  Measured on MI355X (bf16, 1024 and
// 4096 rows, against the rounded-up one-wave instance; outputs identical):
// per token 1.01-1.18x; per 128-group 1.02-1.29x at 3072, 5120, 6144 and
// 7168 channels, but 0.86-1.07x with 64-granule segments (1536, 2560, 3584),
// which keep the one-wave kernel.  Returns false when neither applies.
template <typename T>
bool quant_exact(int64_t group, int ng, dim3 grid, hipStream_t st, const uint16_t* x, uint8_t* q,
                 float* sc, int64_t rows, int64_t xs, int64_t qs) {
  if (ng % kWave != 0) return false;
  const int e = ng / kWave;
  if ((e & (e - 1)) == 0) return false;  // a power of two: the regular instances
  if (group == 8 * (int64_t)ng) {
    switch (e) {
      case 3: act_quant_token_kernel<T, 3, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      case 5: act_quant_token_kernel<T, 5, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      case 6: act_quant_token_kernel<T, 6, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      case 7: act_quant_token_kernel<T, 7, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      case 10: act_quant_token_kernel<T, 10, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      case 12: act_quant_token_kernel<T, 12, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      case 14: act_quant_token_kernel<T, 14, true><<<grid, kBlock, 0, st>>>(x, q, sc, rows, ng, xs, qs); return true;
      default: return false;
    }
  }
  const int gpl = ng % 512 == 0 ? 8 : ng % 256 == 0 ? 4 : ng % 128 == 0 ? 2 : 0;
  if (gpl == 0) return false;
  const int segs = ng / (gpl * kWave);
  const dim3 g2((unsigned)((rows * segs + kRowsPerBlock - 1) / kRowsPerBlock));
  const int lanes = (int)(group / 8);
  const int64_t groups = 8 * (int64_t)ng / group;
  if (gpl == 8) group_go<T, 8, true, true>(lanes, g2, st, x, q, sc, rows, ng, xs, qs, groups, segs);
  else if (gpl == 4) group_go<T, 4, true, true>(lanes, g2, st, x, q, sc, rows, ng, xs, qs, groups, segs);
  else group_go<T, 2, true, true>(lanes, g2, st, x, q, sc, rows, ng, xs, qs, groups, segs);
  return true;
}

template <typename T>
void quant_dispatch(int64_t group, int64_t n, dim3 grid, hipStream_t st, const uint16_t* x,
                    uint8_t* q, float* sc, int64_t rows, int64_t xs, int64_t qs) {
  if (n > 8 * kOneWaveGranules) {
    quant_long<T>(group, n, st, x, q, sc, rows, xs, qs);
    return;
  }
  const int ng = (int)(n / 8);
  if (quant_exact<T>(group, ng, grid, st, x, q, sc, rows, xs, qs)) return;
  const int gpl = quant_gpl(ng);
  const bool full = ng == gpl * kWave;
  switch (gpl) {
    case 1: full ? quant_go<T, 1, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 1, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    case 2: full ? quant_go<T, 2, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 2, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    case 4: full ? quant_go<T, 4, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 4, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    case 8: full ? quant_go<T, 8, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 8, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
    default: full ? quant_go<T, 16, true>(group, n, grid, st, x, q, sc, rows, ng, xs, qs) : quant_go<T, 16, false>(group, n, grid, st, x, q, sc, rows, ng, xs, qs); break;
  }
}

}  // namespace

hipError_t launch_act_quant_fp8(const void* x, uint8_t* q, float* scales, int64_t rows,
                                int64_t n, int64_t group, int64_t xs, int64_t qs, int dtype,
                                hipStream_t stream) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const auto* xp = static_cast<const uint16_t*>(x);
  if (dtype == 1)
    quant_dispatch<F16>(group, n, grid, stream, xp, q, scales, rows, xs, qs);
  else
    quant_dispatch<BF16>(group, n, grid, stream, xp, q, scales, rows, xs, qs);
  return hipGetLastError();
}

}  // namespace qrw
