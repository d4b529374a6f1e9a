// Workgroup -> tile maps of the GEMM and 128x1 quantizer launches.
//
// These are plain integer functions of a workgroup id and the grid, compiled
// for both the host and the device: the kernels call them to find their tile,
// and tests/cpu/tile_map_bijection.cpp runs the very same code on the CPU to
// check that every map is a bijection onto its tiles (a tile computed twice
// or never would otherwise only show as a wrong or missing output block).
//
// The ordering only decides which workgroup computes which tile, never what a
// tile computes, so it has no bearing on the method (Resumen Técnico: Jet-RL,
// "Esquema de Cuantización" fixes the 1x128 / 128x128 / 128x1 groupings and
// the FP8 GEMMs; how their tiles are dealt out is a launch choice).
#pragma once

#include <hip/hip_runtime.h>

namespace fp8bsq {

// The hardware deals workgroup ids round-robin over the 8 XCDs (each with its
// own L2): ids b, b+8, b+16, ... share an XCD.
constexpr int NUM_XCD = 8;

// XCD-aware tile order. Renumber so that each XCD gets a contiguous range of
// logical tiles, then walk logical tiles in groups of GROUP_I tiles along i
// (all j for one group before the next group).
constexpr int GROUP_I = 8;

__host__ __device__ __forceinline__ void map_tile(int bid, int nblk, int tiles_i, int tiles_j, int& ti, int& tj) {
  const int xcd = bid % NUM_XCD, k = bid / NUM_XCD;
  const int per = nblk / NUM_XCD, rem = nblk % NUM_XCD;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + k;
  const int group_span = GROUP_I * tiles_j;
  const int group = logical / group_span;
  const int first_i = group * GROUP_I;
  const int gsize = (tiles_i - first_i) < GROUP_I ? (tiles_i - first_i) : GROUP_I;
  const int in_group = logical - group * group_span;
  ti = first_i + in_group % gsize;
  tj = in_group / gsize;
}

// Chip-wide tile order for long contractions, used by the 8-wavefront tile
// configurations (one workgroup per compute unit, so 256 workgroups run at
// once). The output is cut into supertiles of 16 x 16 tiles; the 256
// workgroups of one round of the chip share a supertile, XCD x taking the
// 4 (i) x 8 (j) block at (4 (x % 4), 8 (x / 4)) of it. Each XCD still works on
// a compact block (12 operand bands for 32 tiles in its L2), and the eight
// XCDs fetch only the supertile's 32 bands between them, the repeats served by
// the last-level cache instead of HBM. Supertiles are walked along j. Tiles
// outside the whole supertiles (a last partial row or column of them) take
// map_tile's order on their own rectangles. Measured on the linears of a
// 32B-parameter model at 32768 tokens: 3-4 % faster where K / 128 >= 64
// (long-contraction DGrad and WGrad), 0.5-1 % slower at K = 5120.
__host__ __device__ __forceinline__ void map_tile_super(int bid, int nblk, int tiles_i, int tiles_j, int& ti,
                                                        int& tj) {
  const int si = tiles_i / 16, sj = tiles_j / 16;
  const int nsup = si * sj;
  if (bid < 256 * nsup) {
    const int xcd = bid % NUM_XCD, k = bid / NUM_XCD;
    const int st = k / 32, s = k % 32;
    ti = (st / sj) * 16 + 4 * (xcd % 4) + (s % 4);
    tj = (st % sj) * 16 + 8 * (xcd / 4) + (s / 4);
    return;
  }
  // bid - 256 nsup has the XCD of bid (256 nsup is a multiple of 8), and so
  // has the offset into the second rectangle (its start 16 si rj is too).
  int r = bid - 256 * nsup;
  const int rj = tiles_j - 16 * sj, ri = tiles_i - 16 * si;
  const int na = 16 * si * rj;    // i < 16 si, j >= 16 sj
  if (r < na) {
    map_tile(r, na, 16 * si, rj, ti, tj);
    tj += 16 * sj;
  } else {                        // i >= 16 si, every j
    r -= na;
    map_tile(r, ri * tiles_j, ri, tiles_j, ti, tj);
    ti += 16 * si;
  }
}
// Contractions of at least this many 128-long blocks use map_tile_super in
// the 8-wavefront configurations.
constexpr int SUPERTILE_MIN_KB = 64;

// Grouped launches: problem g owns the workgroup ids [start[g], start[g+1]).
// Each range starts at a multiple of `align` (the XCD count, or 256 for the
// 8-wavefront tiles so that a problem's supertiles line up with the rounds of
// 256 workgroups the chip runs at once); the ids past a problem's tiles exit
// at once. Returns the total grid size.
__host__ __device__ __forceinline__ int grouped_layout(const int* tiles, int count, int align, int* start) {
  int total = 0;
  for (int g = 0; g < count; ++g) {
    start[g] = total;
    total += (tiles[g] + align - 1) / align * align;
  }
  start[count] = total;
  return total;
}

// The problem that owns workgroup id `bid` (a linear search over at most a
// few dozen starts; the result is uniform over the workgroup).
__host__ __device__ __forceinline__ int grouped_problem(int bid, const int* start, int count) {
  int g = 0;
  while (g + 1 < count && bid >= start[g + 1]) ++g;
  return g;
}

// Workgroup order of the 128x1 and dual quantizers (grid nx token blocks x
// ny channel blocks, n = nx * ny workgroups). Each run of 256 ids is
// renumbered so that every XCD takes 32 consecutive token blocks of one
// channel block, one after another: the 4-byte scale stores of those 32
// workgroups then land in the same 128-byte lines of the transposed scales
// (32 consecutive token blocks of one channel) and, one run later, beside
// each other in the row scales, while the lines are still in that XCD's L2,
// so the lines go out to HBM merged instead of as dozens of partial writes
// (5-9 % faster, same bytes). Ids past the last whole run of 256 keep their
// order.
__host__ __device__ __forceinline__ void token_major_block_of(int bid, int nx, int n, int& mb, int& cbi) {
  int L = bid;
  if (bid < (n / 256) * 256) {
    const int xcd = bid % NUM_XCD, k = bid / NUM_XCD;
    L = (k / 32) * 256 + xcd * 32 + (k % 32);
  }
  mb = L % nx;
  cbi = L / nx;
}

}  // namespace fp8bsq
