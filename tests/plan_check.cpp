// CPU check of the token-row plan used by the RoPE and fused kernels
// (quant_row_workgroup_amd/csrc/qrw_plan.h): every offset a lane can form is
// inside the row, every granule is covered exactly once, rotation pairs sit
// in one item, and the one-table-granule-per-lane shortcut is valid when
// enabled.  Built with g++ by tests/test_plan.py; prints "OK" on success.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "qrw_contig.h"
#include "qrw_plan.h"

using namespace qrw;

static int fails = 0;
#define CHECK(c, ...)                 \
  do {                                \
    if (!(c)) {                       \
      if (fails < 20) {               \
        std::printf(__VA_ARGS__);     \
        std::printf("\n");            \
      }                               \
      ++fails;                        \
    }                                 \
  } while (0)

static void check_shape(int heads, int head_dim, int rope_dim, bool neox, int kmax) {
  RowPlan p = make_plan(heads, head_dim, rope_dim);
  const int n = heads * head_dim;
  std::vector<int> cover(n / 8, 0);
  // the kernels visit items lane + 64*i for i < K (fused: one pass, K = kmax;
  // RoPE: passes of 64*K) -- visit a generous superset of indices
  const int limit = p.n_items + 64 * kmax;
  for (int it = 0; it < limit; ++it) {
    int a, b, s;
    int kind = item_offsets(p, it, neox, a, b, s);
    if (it >= p.n_items) {
      CHECK(kind == kItemNone, "item %d beyond n_items has kind %d", it, kind);
      continue;
    }
    CHECK(kind != kItemNone, "item %d < n_items=%d is empty (h=%d D=%d R=%d)", it, p.n_items,
          heads, head_dim, rope_dim);
    CHECK(a >= 0 && a % 8 == 0 && a + 8 <= n, "A out of row: it=%d a=%d n=%d", it, a, n);
    if (b >= 0) CHECK(b % 8 == 0 && b + 8 <= n, "B out of row: it=%d b=%d n=%d", it, b, n);
    if (a >= 0 && a + 8 <= n) cover[a / 8]++;
    if (b >= 0 && b + 8 <= n) cover[b / 8]++;
    if (kind == kItemRope) {
      CHECK(b >= 0, "rope item without B");
      CHECK(s >= 0 && s < p.gph && 8 * s + 8 <= rope_dim / 2, "table granule out of range");
      const int h = a / head_dim;
      const int off = a - h * head_dim;  // offset inside the head
      const int start = head_dim - rope_dim;
      CHECK(off >= start, "rope granule before the span");
      CHECK(b / head_dim == h, "pair crosses heads");
      if (neox) {
        CHECK(off - start == 8 * s && b - a == rope_dim / 2, "neox pairing wrong");
      } else {
        CHECK(off - start == 16 * s && b - a == 8, "interleaved pairing wrong");
      }
      if (p.lane_hoist) CHECK(s == (it % 64) % p.gph, "lane hoist invalid at it=%d", it);
    } else if (kind == kItemPlain) {
      const int off = a % head_dim;
      CHECK(off < head_dim - rope_dim, "plain granule inside the span");
      if (b >= 0) CHECK(b % head_dim < head_dim - rope_dim, "plain B inside the span");
    }
  }
  for (int g = 0; g < n / 8; ++g)
    CHECK(cover[g] == 1, "granule %d covered %d times (h=%d D=%d R=%d)", g, cover[g], heads,
          head_dim, rope_dim);
}

// The contiguous lane mapping (qrw_contig.h) of the RoPE and tail-rotation
// kernels: lane l owns granules l + 64 g, g < G.  Checks every granule is
// owned once and in the row; a rotating granule's position in its span is the
// lane's fixed position (so one table granule per lane is right) and its
// table entries lie in the table row; the NeoX partner granule is lane
// l ^ rope_dim/16 of the same step, in the same head's span at the partner
// position; granules outside every span are never rotated.
static int contig_checked = 0;
static void check_contig(int heads, int head_dim, int rope_dim, int g_blocks) {
  const int n = heads * head_dim;
  if (g_blocks == 0) return;
  ++contig_checked;
  CHECK(n == 512 * g_blocks, "contig row %d is not 512*%d", n, g_blocks);
  const int hg = head_dim / 8, hg_mask = hg - 1, s0 = (head_dim - rope_dim) / 8;
  const int span_len = rope_dim / 8, xr = rope_dim / 16, half = rope_dim / 2;
  std::vector<int> cover(n / 8, 0);
  for (int lane = 0; lane < 64; ++lane) {
    const int jl = contig_span_pos(lane, hg_mask, s0);
    for (int g = 0; g < g_blocks; ++g) {
      const int gi = 64 * g + lane;
      CHECK(8 * gi + 8 <= n, "contig granule %d out of row %d", gi, n);
      if (8 * gi + 8 <= n) cover[gi]++;
      const int j = gi % hg;  // position inside the head
      const bool in_span = j >= s0;
      CHECK(contig_rotates(gi, hg_mask, s0) == in_span, "rotation test wrong at gi=%d", gi);
      if (!in_span) continue;
      CHECK(j - s0 == jl, "span position %d != lane's %d (H=%d D=%d R=%d lane=%d g=%d)", j - s0,
            jl, heads, head_dim, rope_dim, lane, g);
      CHECK(jl >= 0 && jl < span_len, "span position %d out of [0,%d)", jl, span_len);
      // NeoX: table granule jl mod xr, 8 entries; interleaved: entries 4 jl .. 4 jl + 3
      CHECK(8 * (jl % xr) + 8 <= half, "neox table granule out of the row");
      CHECK(4 * jl + 4 <= half, "interleaved table entries out of the row");
      const int partner = gi ^ xr;
      CHECK(partner == 64 * g + (lane ^ xr), "neox partner not lane ^ xr in the same step");
      CHECK(partner / hg == gi / hg && partner % hg >= s0 && partner % hg - s0 == (jl ^ xr),
            "neox partner outside the head's span (gi=%d)", gi);
    }
  }
  for (int k = 0; k < n / 8; ++k) CHECK(cover[k] == 1, "contig granule %d owned %d times", k, cover[k]);
}

int main() {
  // exhaustive: the largest item count over every accepted shape fits one
  // fused launch (64 lanes x 8 items)
  int worst = 0;
  for (int D = 8; D <= 8192; D += 8)
    for (int R = 16; R <= D; R += 16)
      for (int H = 1; H * D <= 8192; ++H) {
        RowPlan p = make_plan(H, D, R);
        if (p.n_items > worst) worst = p.n_items;
      }
  CHECK(worst <= 512, "an accepted shape needs %d items > 512", worst);
  std::printf("max items per token: %d\n", worst);
  // fast-division identity over the whole range used
  for (int d = 1; d < 1100; ++d) {
    FastDiv f = make_fastdiv(d);
    for (int x = 0; x < 4200; ++x) CHECK(fastdiv(f, x) == x / d, "fastdiv %d / %d", x, d);
  }
  // coverage of a spread of shapes, including the benchmark ones
  const int shapes[][3] = {{32, 128, 128}, {1, 4096, 128}, {32, 128, 64}, {8, 64, 16},
                           {3, 48, 32},    {1, 8192, 16},  {64, 128, 128}, {5, 24, 16},
                           {2, 8, 8},      {7, 96, 96},    {1, 16, 16},    {4, 256, 128},
                           {1, 1000, 16},  {13, 40, 32},   {16, 512, 512}, {2, 4096, 4096},
                           {1, 8184, 16},  {11, 72, 48}};
  for (auto& s : shapes) {
    if (s[2] % 16 != 0) continue;
    for (int nx = 0; nx < 2; ++nx) check_shape(s[0], s[1], s[2], nx == 1, 8);
  }
  // a random sweep
  std::srand(1234);
  for (int k = 0; k < 3000; ++k) {
    int D = 8 * (1 + std::rand() % 256);
    if (D < 16) D = 16;
    int R = 16 * (1 + std::rand() % (D / 16));
    int Hmax = 8192 / D;
    int H = 1 + std::rand() % (Hmax < 40 ? Hmax : 40);
    check_shape(H, D, R, (k & 1) != 0, 8);
  }
  // the contiguous mapping over every shape it accepts (RoPE) and the tail
  // kernel's shapes (rope_dim < head_dim, up to 8 blocks), and its refusals
  for (int nx = 0; nx < 2; ++nx)
    for (int D = 16; D <= 8192; D *= 2)
      for (int R = 16; R <= D && R <= 512; R *= 2)
        for (int H = 1; H * D <= 16384; ++H) {
          const bool neox = nx == 1;
          const int g = rope_contig_blocks(H, D, R, neox);
          const int blocks = (H * D) % 512 == 0 ? (H * D) / 512 : 0;
          const bool p2 = blocks == 1 || blocks == 2 || blocks == 4 || blocks == 8 || blocks == 16;
          const bool odd = blocks == 3 || blocks == 5 || blocks == 6 || blocks == 7 ||
                           blocks == 10 || blocks == 12 || blocks == 14;
          const bool want = R <= 256 && (p2 || (odd && (D == 64 || D == 128) && (!neox || R == D)));
          CHECK((g != 0) == want, "rope_contig_blocks(%d,%d,%d,%d) = %d", H, D, R, (int)neox, g);
          CHECK(g == 0 || g == blocks, "rope_contig_blocks(%d,%d,%d) = %d blocks", H, D, R, g);
          check_contig(H, D, R, g);
        }
  CHECK(rope_contig_blocks(32, 192, 64, true) == 0 && rope_contig_blocks(4, 128, 24, false) == 0 &&
            rope_contig_blocks(40, 128, 64, true) == 0 && rope_contig_blocks(9, 128, 128, true) == 0,
        "non-power-of-two heads, odd rows rotating part of a NeoX head, rows of 1152 channels "
        "must take the item kernel");
  CHECK(rope_contig_blocks(40, 128, 128, true) == 10 && rope_contig_blocks(40, 128, 64, false) == 10,
        "40 heads of 128 take the contiguous kernel");
  std::printf("contiguous mapping: %d shapes\n", contig_checked);
  if (fails) {
    std::printf("FAILED %d checks\n", fails);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
