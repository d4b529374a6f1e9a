// CPU check that the launch maps of the GEMM and 128x1 quantizer kernels are
// bijections: every tile (or token x channel block) is owned by exactly one
// workgroup id, and no id maps outside the grid.
//
// It includes the kernels' own header (csrc/tile_map.h, whose functions are
// compiled for host and device) and runs them on the CPU, so the code checked
// is the code the kernels execute. Built host-only with hipcc by
// tests/test_tile_maps.py.
//
// Input (stdin), one case per line:
//   plain  TI TJ                 map_tile over a TI x TJ tile grid
//   super  TI TJ                 map_tile_super over a TI x TJ tile grid
//   all    N                     plain and super for every grid up to N x N
//   group  ALIGN G  TI TJ S ...  a grouped launch of G problems (TI x TJ tiles,
//                                S = 1 if the problem uses map_tile_super),
//                                ranges aligned to ALIGN workgroup ids
//   quant  NX NY                 token_major_block_of over NX x NY blocks
// Output: one "ok <kind> <ids>" line per case, or "FAIL ..." and exit code 1.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../fp8_block_scaled_quantize_amd/csrc/tile_map.h"

using namespace fp8bsq;

static int failures = 0;

static bool fail(const char* what, int a, int b, int c, int d) {
  std::printf("FAIL %s %d %d %d %d\n", what, a, b, c, d);
  ++failures;
  return false;
}

// Every id in [0, TI*TJ) maps into the grid and every tile is hit once.
static bool check_grid(bool super, int TI, int TJ) {
  const int n = TI * TJ;
  std::vector<int> hits(n, 0);
  for (int bid = 0; bid < n; ++bid) {
    int ti = -1, tj = -1;
    if (super) map_tile_super(bid, n, TI, TJ, ti, tj);
    else map_tile(bid, n, TI, TJ, ti, tj);
    if (ti < 0 || ti >= TI || tj < 0 || tj >= TJ) return fail(super ? "super-range" : "plain-range", TI, TJ, bid, ti);
    if (hits[ti * TJ + tj]++) return fail(super ? "super-dup" : "plain-dup", TI, TJ, ti, tj);
  }
  return true;
}

int main() {
  char kind[16];
  while (std::scanf("%15s", kind) == 1) {
    if (!std::strcmp(kind, "plain") || !std::strcmp(kind, "super")) {
      int TI, TJ;
      if (std::scanf("%d %d", &TI, &TJ) != 2) return 2;
      if (check_grid(kind[0] == 's', TI, TJ)) std::printf("ok %s %d\n", kind, TI * TJ);
    } else if (!std::strcmp(kind, "all")) {
      int N;
      if (std::scanf("%d", &N) != 1) return 2;
      long ids = 0;
      bool ok = true;
      for (int TI = 1; TI <= N; ++TI)
        for (int TJ = 1; TJ <= N; ++TJ) {
          ok = check_grid(false, TI, TJ) && ok;
          ok = check_grid(true, TI, TJ) && ok;
          ids += 2L * TI * TJ;
        }
      if (ok) std::printf("ok all %ld\n", ids);
    } else if (!std::strcmp(kind, "group")) {
      int align, G;
      if (std::scanf("%d %d", &align, &G) != 2 || G < 1 || G > 64) return 2;
      std::vector<int> ti_n(G), tj_n(G), sup(G), tiles(G), start(G + 1);
      for (int g = 0; g < G; ++g) {
        if (std::scanf("%d %d %d", &ti_n[g], &tj_n[g], &sup[g]) != 3) return 2;
        tiles[g] = ti_n[g] * tj_n[g];
      }
      const int total = grouped_layout(tiles.data(), G, align, start.data());
      std::vector<std::vector<int>> hits(G);
      for (int g = 0; g < G; ++g) {
        hits[g].assign(tiles[g], 0);
        if (start[g] % align) fail("group-align", g, start[g], align, 0);
      }
      bool ok = failures == 0;
      for (int bid = 0; bid < total && ok; ++bid) {
        const int g = grouped_problem(bid, start.data(), G);
        if (g < 0 || g >= G || bid < start[g] || bid >= start[g + 1]) { ok = fail("group-owner", bid, g, 0, 0); break; }
        const int local = bid - start[g];
        if (local >= tiles[g]) continue;   // padding id: the kernel returns at once
        int ti = -1, tj = -1;
        if (sup[g]) map_tile_super(local, tiles[g], ti_n[g], tj_n[g], ti, tj);
        else map_tile(local, tiles[g], ti_n[g], tj_n[g], ti, tj);
        if (ti < 0 || ti >= ti_n[g] || tj < 0 || tj >= tj_n[g]) { ok = fail("group-range", g, local, ti, tj); break; }
        if (hits[g][ti * tj_n[g] + tj]++) { ok = fail("group-dup", g, ti, tj, 0); break; }
      }
      for (int g = 0; g < G && ok; ++g)
        for (int t = 0; t < tiles[g]; ++t)
          if (hits[g][t] != 1) { ok = fail("group-miss", g, t, hits[g][t], 0); break; }
      if (ok) std::printf("ok group %d\n", total);
    } else if (!std::strcmp(kind, "quant")) {
      int NX, NY;
      if (std::scanf("%d %d", &NX, &NY) != 2) return 2;
      const int n = NX * NY;
      std::vector<int> hits(n, 0);
      bool ok = true;
      for (int bid = 0; bid < n; ++bid) {
        int mb = -1, cb = -1;
        token_major_block_of(bid, NX, n, mb, cb);
        if (mb < 0 || mb >= NX || cb < 0 || cb >= NY) { ok = fail("quant-range", NX, NY, bid, mb); break; }
        if (hits[cb * NX + mb]++) { ok = fail("quant-dup", NX, NY, mb, cb); break; }
      }
      if (ok) std::printf("ok quant %d\n", n);
    } else {
      std::printf("FAIL unknown-case %s 0 0 0 0\n", kind);
      return 2;
    }
  }
  return failures ? 1 : 0;
}
