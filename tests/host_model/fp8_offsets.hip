// Host-side model of the fp8 64-row tile's operand loads (CPU only; no GPU
// call is made).  For every unit — planned and decoded with the kernels' own
// plan_units / decode_unit_seg from the per-segment tile table — and every
// 128-K step, it forms each lane's voffset and soffset the way small_unit_fp8
// does (with the kernel's fp8_a_voff / fp8_b_voff half-step rule) and checks
// that every load the buffer range check lets through stays inside its
// allocation.  It also decodes every unit through the tile-list form
// (decode_unit_plain over the list build_tiles_kernel writes for the same
// segments) and counts the units on which the two decoders disagree.
//
// Usage: fp8_offsets <mode: up|down> <K> <Nn> <rows per expert...>
// Prints "units=U checked=C oob=O nohalf_oob=H list_mismatch=M kind0_mismatch=M0
// cover_bad=B": O loads past their allocation with the half-step rule, H without
// it; B cells of (row, column tile, K step) that the bf16 units of tile kinds 0,
// 2, 3 and 4 cover other than once.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../mixture_experts_layer_histogram_amd/csrc/gemm_tile.h"

using namespace moe;

struct Count {
  long long units = 0, checked = 0, oob = 0, mismatch = 0;
};

// The table build_seg_table writes (exclusive prefix counts of seg_tiles; kinds 3
// and 4 resolved to 0 or 2 with the kernels' choose_tail_kind).
static SegTable seg_table(const std::vector<int>& offs, int kind, int n_ntiles = 0, int G = 256,
                          bool attach = false) {
  SegTable t{};
  const int E = (int)offs.size() - 1;
  if (kind >= 3) {
    long long c0 = 0, c2 = 0;
    for (int e = 0; e < E; ++e) {
      int b0, b2, s_;
      seg_tiles(offs[e + 1] - offs[e], 0, b0, s_);
      seg_tiles(offs[e + 1] - offs[e], 2, b2, s_);
      c0 += b0;
      c2 += b2;
    }
    kind = choose_tail_kind(c0 * n_ntiles, c2 * n_ntiles, G, kind == 4);
  }
  if (attach && kind == 0) kind = 5;
  t.kind = kind;
  int b = 0, sm = 0;
  for (int e = 0; e < E; ++e) {
    int nb, ns;
    seg_tiles(offs[e + 1] - offs[e], kind, nb, ns);
    t.off[e] = offs[e]; t.pb[e] = b; t.ps[e] = sm;
    b += nb; sm += ns;
  }
  t.off[E] = offs[E]; t.pb[E] = b; t.ps[E] = sm;
  return t;
}

static Count run(bool up, int K, int Nn, const std::vector<int>& seg_rows, bool half_rule) {
  const int E = (int)seg_rows.size();
  const int G = 256;                                // one workgroup per CU, a multiple of 8
  const int KT = K / 64;
  const int cols_per_tile = up ? 128 : 256;         // SwiGLU up: 128 W1 + 128 W3 columns per tile
  const int n_ntiles = (Nn + cols_per_tile - 1) / cols_per_tile;
  // 64-row tile list (kind 1): ceil(rows / 64) tiles per segment
  std::vector<int> offs(E + 1, 0);
  for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + seg_rows[e];
  std::vector<int32_t> tiles(4);
  int nt = 0;
  for (int e = 0; e < E; ++e) {
    const int n = (seg_rows[e] + 63) / 64;
    for (int i = 0; i < n; ++i) {
      const int r0 = offs[e] + 64 * i, r1 = std::min(offs[e + 1], r0 + 64);
      const int32_t ent[8] = {e, r0, r1, nt - i, n, 0, 0, 0};
      tiles.insert(tiles.end(), ent, ent + 8);
      ++nt;
    }
  }
  tiles[0] = nt;
  const long long kept = offs[E];
  const long long N = up ? kept : 0;                // gather: one token row per kept slot (k = 1 model)
  const long long rowbytes = 2LL * K;
  const long long a_alloc = (up ? N : kept) * rowbytes;   // x (up) or h (down) rows written / held
  const long long b_alloc = (long long)E * Nn * K;        // fp8 weights
  const SegTable table = seg_table(offs, 1);
  const UnitPlan plan = plan_units(table.ps[E] * n_ntiles, G, KT);
  Count c;
  for (int u = 0; u < plan.units(); ++u) {
    const Unit w = decode_unit_seg(table, E, false, plan, u, n_ntiles, KT, cols_per_tile);
    const Unit wl = decode_unit_plain(tiles.data(), plan, u, n_ntiles, KT, cols_per_tile);
    if (w.seg != wl.seg || w.r0 != wl.r0 || w.r1 != wl.r1 || w.n0 != wl.n0 || w.kt0 != wl.kt0 || w.kt1 != wl.kt1 ||
        w.slot != wl.slot)
      ++c.mismatch;
    ++c.units;
    const int n64 = w.kt1 - w.kt0, nst = (n64 + 1) / 2;
    const long long a_base = up ? 0 : (long long)w.r0 * rowbytes;
    const long long a_recs = up ? N * rowbytes : (long long)(w.r1 - w.r0) * rowbytes;
    const int nb_rows = std::min(cols_per_tile, Nn - w.n0);
    const long long b_base = (long long)w.seg * Nn * K + (long long)w.n0 * K;
    const long long b_recs = (long long)nb_rows * K;
    for (int j = 0; j < nst; ++j) {
      const int k64 = w.kt0 + 2 * j;
      const bool half = half_rule && (2 * j + 1 >= n64);
      for (int wn = 0; wn < 4; ++wn)
        for (int lane = 0; lane < 64; ++lane) {
          for (int ua = 0; ua < 2; ++ua) {
            const int row = 16 * wn + 8 * ua + (lane >> 3);
            const int chunk = (lane & 7) ^ swz8(row);
            int voff;
            if (up) {   // gather: row r of the expert order is token r (k = 1)
              const int r = w.r0 + row;
              voff = (r < w.r1 ? r * (int)rowbytes : kOobOffset) + chunk * 16;
            } else {
              voff = row * (int)rowbytes + chunk * 16;
            }
            for (int hf = 0; hf < 2; ++hf) {
              const long long v = fp8_a_voff(voff, hf, half);
              const long long so = (long long)(k64 + hf) * 128;
              if (v >= a_recs) continue;          // range check: reads zero, no access
              ++c.checked;
              if (a_base + v + so + 16 > a_alloc) ++c.oob;
            }
          }
          for (int ub = 0; ub < 8; ++ub) {
            const int row = 64 * wn + 8 * ub + (lane >> 3);
            const int chunk = (lane & 7) ^ swz8(row);
            const int voff = (up ? (row & 127) : row) * K + chunk * 16;
            const long long v = fp8_b_voff(voff, chunk, half);
            const long long so = (long long)k64 * 64;
            if (v >= b_recs) continue;
            ++c.checked;
            if (b_base + v + so + 16 > b_alloc) ++c.oob;
          }
        }
    }
  }
  return c;
}

// Kind 0 (the bf16 path: 256-row tiles, a 256-row tile for tails of at least
// kBigTailMin rows, 64-row tiles for the rest): both lists in build_tiles_kernel's
// layout, and the units of each decoded both ways; returns the disagreements.
static long long kind0_mismatch(int K, int Nn, int cols_per_tile, const std::vector<int>& seg_rows) {
  const int E = (int)seg_rows.size(), KT = K / 64, G = 256;
  const int n_ntiles = (Nn + cols_per_tile - 1) / cols_per_tile;
  std::vector<int> offs(E + 1, 0);
  for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + seg_rows[e];
  std::vector<int32_t> big(4), small(4);
  int nbt = 0, nst = 0;
  for (int e = 0; e < E; ++e) {
    int nb, ns;
    seg_tiles(seg_rows[e], 0, nb, ns);
    const int split = std::min(offs[e + 1], offs[e] + nb * 256);
    for (int i = 0; i < nb; ++i) {
      const int32_t ent[8] = {e, offs[e] + 256 * i, std::min(offs[e + 1], offs[e] + 256 * (i + 1)), nbt - i, nb,
                              0, 0, 0};
      big.insert(big.end(), ent, ent + 8);
      ++nbt;
    }
    for (int i = 0; i < ns; ++i) {
      const int32_t ent[8] = {e, split + 64 * i, std::min(offs[e + 1], split + 64 * (i + 1)), nst - i, ns, 0, 0, 0};
      small.insert(small.end(), ent, ent + 8);
      ++nst;
    }
  }
  big[0] = nbt;
  small[0] = nst;
  const SegTable t = seg_table(offs, 0);
  long long bad = 0;
  for (int kind = 0; kind < 2; ++kind) {
    const bool isbig = kind == 0;
    const UnitPlan plan = plan_units((isbig ? nbt : nst) * n_ntiles, G, KT);
    for (int u = 0; u < plan.units(); ++u) {
      const Unit a = decode_unit_seg(t, E, isbig, plan, u, n_ntiles, KT, cols_per_tile);
      const Unit b = decode_unit_plain((isbig ? big : small).data(), plan, u, n_ntiles, KT, cols_per_tile);
      bad += a.seg != b.seg || a.r0 != b.r0 || a.r1 != b.r1 || a.n0 != b.n0 || a.kt0 != b.kt0 || a.kt1 != b.kt1 ||
             a.slot != b.slot;
    }
  }
  return bad;
}

// Every kind of the bf16 path (0, 2, and the chosen one for 3 and 4): the
// 256-row and 64-row units, decoded from the table, cover every (row, output
// column tile, K step) of every segment exactly once and nothing outside the
// segments; returns the number of cells covered other than once.
static long long cover_bad(int K, int Nn, int cols_per_tile, const std::vector<int>& seg_rows, int kind,
                           bool attach = false) {
  const int E = (int)seg_rows.size(), KT = K / 64, G = 256;
  const int n_ntiles = (Nn + cols_per_tile - 1) / cols_per_tile;
  std::vector<int> offs(E + 1, 0);
  for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + seg_rows[e];
  const SegTable t = seg_table(offs, kind, n_ntiles, G, attach);
  const int R = offs[E];
  std::vector<unsigned char> hits((size_t)R * n_ntiles * KT, 0);
  long long bad = 0;
  for (int big = 0; big < 2; ++big) {
    const UnitPlan plan = plan_units((big ? t.pb[E] : t.ps[E]) * n_ntiles, G, KT);
    // the units as the kernels reach them: workgroup q of XCD x walks its XCD's slices
    std::vector<int> order;
    for (int x = 0; x < kXcds; ++x) {
      const XcdSlice xs = xcd_slice(plan, x);
      for (int q = 0; q < G / kXcds; ++q)
        for (int i = q; i < xs.fc + xs.pc; i += G / kXcds) order.push_back(xcd_unit(plan, xs, i));
    }
    if ((long long)order.size() != plan.units()) bad += 1000000;
    for (int u : order) {
      const Unit w = decode_unit_seg(t, E, big != 0, plan, u, n_ntiles, KT, cols_per_tile);
      if (w.r1 - w.r0 > (big ? 256 : 64) || w.r0 < offs[w.seg] || w.r1 > offs[w.seg + 1] || w.r0 >= w.r1) {
        ++bad;
        continue;
      }
      const int j = w.n0 / cols_per_tile;
      for (int r = w.r0; r < w.r1; ++r)
        for (int kt = w.kt0; kt < w.kt1; ++kt) ++hits[((size_t)r * n_ntiles + j) * KT + kt];
      if (w.x1 > w.x0) {   // attached tail rows: only on whole 256-row tiles, at most 32, in the same segment
        if (!big || w.r1 - w.r0 != 256 || w.x1 - w.x0 > kAttachRows || w.x0 < offs[w.seg] ||
            w.x1 > offs[w.seg + 1]) {
          ++bad;
          continue;
        }
        for (int r = w.x0; r < w.x1; ++r)
          for (int kt = w.kt0; kt < w.kt1; ++kt) ++hits[((size_t)r * n_ntiles + j) * KT + kt];
      }
    }
  }
  for (unsigned char h : hits) bad += h != 1;
  return bad;
}

int main(int argc, char** argv) {
  if (argc < 5) {
    std::fprintf(stderr, "usage: %s up|down K Nn rows...\n", argv[0]);
    return 2;
  }
  const bool up = argv[1][0] == 'u';
  const int K = std::atoi(argv[2]), Nn = std::atoi(argv[3]);
  std::vector<int> rows;
  for (int i = 4; i < argc; ++i) rows.push_back(std::atoi(argv[i]));
  const Count a = run(up, K, Nn, rows, true), b = run(up, K, Nn, rows, false);
  const int cpt = up ? 128 : 256;
  const long long m0 = kind0_mismatch(K, Nn, cpt, rows);
  long long cov = 0;
  for (int kind : {0, 2, 3, 4}) cov += cover_bad(K, Nn, cpt, rows, kind) + cover_bad(K, Nn, cpt, rows, kind, true);
  long long attached = 0;   // rows the attaching table hands to 256-row units (the cases must exercise it)
  {
    std::vector<int> offs(rows.size() + 1, 0);
    for (size_t e = 0; e < rows.size(); ++e) offs[e + 1] = offs[e] + rows[e];
    const SegTable t = seg_table(offs, 0, 1, 256, true);
    for (size_t e = 0; e < rows.size(); ++e) attached += t.kind == 5 ? attach_rows(rows[e]) : 0;
  }
  int auto_kind;   // the kind the forward kernels resolve for these segments (rule 3 up, 4 down, attaching)
  {
    std::vector<int> offs(rows.size() + 1, 0);
    for (size_t e = 0; e < rows.size(); ++e) offs[e + 1] = offs[e] + rows[e];
    auto_kind = seg_table(offs, up ? 3 : 4, (Nn + cpt - 1) / cpt, 256, true).kind;
  }
  std::printf("units=%lld checked=%lld oob=%lld nohalf_oob=%lld list_mismatch=%lld kind0_mismatch=%lld "
              "cover_bad=%lld attached=%lld auto_kind=%d\n", a.units, a.checked, a.oob, b.oob, a.mismatch, m0, cov,
              attached, auto_kind);
  return 0;
}
