// Scale-aware FP8 GEMMs on gfx950 MFMA: forward, DGrad and WGrad.
//
// Source: Resumen Técnico: Jet-RL (gist.science), "Esquema de Cuantización":
// the linear layers are FP8 GEMMs -- forward on 1x128-grouped activations and
// 128x128-block weights, DGrad and WGrad in FP8 as well, WGrad with both
// operands grouped along the tokens (1x128 / 128x1).
//
// One kernel family serves all three roles. It computes, for operands P [I, K]
// and Q [J, K] (both K-contiguous E4M3) with one fp32 scale per 128-long
// K block,
//     out[j][i] = bf16( sum_kb  ps(i, kb) * qs(j, kb) * sum_{k in kb} P[i,k] * Q[j,k] )
// and writes the columns i < Iout of out as a row-major [J, Iout] bf16 matrix.
//   forward: P = Wq [Np, Kp] (block scales), Q = Xq [M, Kp]   -> out = Y  [M, N]
//   DGrad  : P = Wq^T [Kp, Np] (block scales, read transposed), Q = dYq [M, Np] -> dX [M, K]
//   WGrad  : P = Xq^T [K, Mp] (row scales), Q = dYq^T [N, Mp] -> dW [N, K]
// (Np, Kp, Mp: N, K, M rounded up to 128; the code tensors are padded with +0
// codes along their grouped dimensions, so the contraction always runs over
// whole 128-long blocks and the block-scaled P always has whole 128-row
// blocks; a partial last block of N or K only masks the stored columns.)
//
// Each 128-long K block is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16
// output tile, so the block's partial sum comes out of a single MFMA with a
// zero accumulator and is promoted into the fp32 running sum,
// acc += partial * ps * qs: one FMA per element where the P scale is per
// 128x128 block (forward, DGrad), a multiply and an FMA where both scales are
// per row (WGrad). In the MFMA result layout a lane holds four consecutive i
// of one j, so the Q scale is one value per lane and a block P scale is
// uniform over the wavefront.
//
// Tiles: a workgroup owns a BI x BJ output tile and walks K in 128-byte steps.
// Both operand tiles of a step are staged in LDS (two to four stages) with
// their 16-byte chunks XOR-swizzled by row so that the MFMA fragment reads are
// free of bank conflicts. Workgroups are mapped to tiles so that each XCD works on
// a compact band of the output (its own L2), in groups along i; for long
// contractions the 8-wavefront configurations also keep the eight XCDs inside one
// 16 x 16 block of tiles at a time (shared operand bands in the last-level
// cache).
#include "device_common.h"
#include "launch.h"
#include "tile_map.h"

#include <type_traits>

namespace fp8bsq {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct GemmParams {
  const uint8_t* P;
  const float* Ps;
  const uint8_t* Q;
  const float* Qs;
  uint16_t* out;
  int I, J, K, Kb;
  int Iout, ldo;     // columns i < Iout of out are stored, rows ldo elements apart
  int ps_ib, ps_kb;  // block P scale of (i, kb) at Ps[(i / 128) * ps_ib + kb * ps_kb]
  int tiles_i, tiles_j;
};

template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST_ = 2>
struct GemmCfg {
  static constexpr int NST = NST_;                               // LDS stages (K steps in flight + 1)
  static constexpr int WI = SI * 16, WJ = SJ * 16;              // wavefront tile
  static constexpr int BI = WAVES_I * WI, BJ = WAVES_J * WJ;    // workgroup tile
  static constexpr int NT = 64 * WAVES_I * WAVES_J;
  static constexpr int P_LOADS = BI * 8 / NT;                    // 16-byte loads per thread
  static constexpr int Q_LOADS = BJ * 8 / NT;
  static constexpr int ROWSC = BJ + (PS_ROW ? BI : 0);          // per-row scales per K step
  static constexpr int BLKSC = PS_ROW ? 0 : (BI + 127) / 128;    // 128x128-block P scales per K step
  static constexpr int BLKSC_PAD = BLKSC > 0 ? BLKSC : 1;
  static constexpr int TILE_BYTES = (BI + BJ) * 128;
  static_assert(BI * 8 % NT == 0 && BJ * 8 % NT == 0, "loads must divide evenly");
  static constexpr int ROW_PASSES = (ROWSC + NT - 1) / NT;      // per-row scales per thread
  static_assert(BLKSC <= 64 && BJ % 64 == 0 && NT % 64 == 0, "scale lanes");
  static_assert(PS_ROW || (128 % WI == 0), "a block-scaled wavefront must sit inside one 128-row block");
  static_assert(BI % 64 == 0 && (BI >= 128 || 128 % BI == 0), "a workgroup's P rows sit in whole 128-row blocks or inside one");
};

// Byte offset of 16-byte chunk `chunk` of tile row `row` (rows are 128 bytes).
// The chunk index is XORed with f(row) = (row & 7) ^ ((row >> 3) & 1), so that
// the MFMA fragment reads (one 16-byte chunk from each of 16 consecutive rows
// per 16 lanes) hit distinct banks whether the LDS serves 8 lanes x 16 bytes
// or 16 lanes x 16 bytes per clock: any 8 aligned consecutive rows get 8
// distinct chunk slots, and the even and the odd rows of any 16 aligned
// consecutive rows each get 8 distinct slots.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_key(row)) << 4); }

// One workgroup's output tile: tile number `bid` of the `nblk` tiles of
// problem p (a plain launch passes its block index and grid size; a grouped
// launch its block's offset within the problem).
// V4: K/128 is a multiple of 4 (for every problem of a grouped launch), so
// each row's scales for 4 consecutive K steps are one aligned 16-byte copy.
template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST, bool CLAMP, bool V4>
__device__ __forceinline__ void gemm_body(const GemmParams& p, int bid, int nblk) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses LDS address-space casts, device pass only
  using C = GemmCfg<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST>;
  __shared__ __align__(16) uint8_t tiles[NST][C::TILE_BYTES];
  // Per-row scales come in groups of 4 K steps, [row][4], double-buffered by
  // group; block P scales come per K step.
  __shared__ __align__(16) float rowsc[2][C::ROWSC * 4];
  __shared__ __align__(16) float blksc[NST][C::BLKSC_PAD];
  // The block-scaled roles (X W^T, dY W) prefetch each K step's tile rows
  // into L2 one step before their LDS copies go out; for the row-scaled role
  // (dY^T X, rows a full token count apart) this measured slower.
  constexpr bool PF_L2 = !PS_ROW && C::BI + C::BJ == C::NT;
  // Landing area of the L2 prefetch copies (never read).
  __shared__ __align__(16) uint32_t pf_sink[PF_L2 ? C::NT : 1];

  const uint32_t tiles_lds = lds_addr(&tiles[0][0]);
  const uint32_t rowsc_lds = lds_addr(&rowsc[0][0]);
  const uint32_t blksc_lds = lds_addr(&blksc[0][0]);
  const uint32_t sink_lds = lds_addr(&pf_sink[0]);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wi = wave % WAVES_I, wj = wave / WAVES_I;
  const int g = lane >> 4, r16 = lane & 15;

  int ti, tj;
  if (C::NT == 512 && p.Kb >= SUPERTILE_MIN_KB)
    map_tile_super(bid, nblk, p.tiles_i, p.tiles_j, ti, tj);
  else
    map_tile(bid, nblk, p.tiles_i, p.tiles_j, ti, tj);
  // The last tile along a dimension is shifted back to end at the edge, so
  // every row it loads exists; where it overlaps its neighbour both compute
  // and store the same values. Only a dimension smaller than one tile (the
  // CLAMP instantiation) needs clamped rows, whose outputs are never stored.
  const int i0 = p.I >= C::BI ? min(ti * C::BI, p.I - C::BI) : 0;
  const int j0 = p.J >= C::BJ ? min(tj * C::BJ, p.J - C::BJ) : 0;
  const int prows = min(p.I - i0, C::BI);
  const int qrows = min(p.J - j0, C::BJ);

  // ---- operand tiles. One DMA instruction moves one 8-row slab (1 KB), lane
  //      L landing at byte 16L. Lane L therefore fetches the global chunk that
  //      the swizzled layout keeps at that spot: row 8n + L/8 of slab n,
  //      logical chunk (L%8) ^ swz_key(row), where swz_key(row) = (L/8) ^ (n & 1). ----
  constexpr int P_INSTR = C::BI / 8 / (C::NT / 64);   // slabs per wavefront
  constexpr int Q_INSTR = C::BJ / 8 / (C::NT / 64);
  static_assert(P_INSTR * 8 * (C::NT / 64) == C::BI && Q_INSTR * 8 * (C::NT / 64) == C::BJ, "tile rows per wave");
  const int lrow = lane >> 3;
  const uint32_t loff0 = (uint32_t)(lrow * p.K + (((lane & 7) ^ lrow) << 4));
  const uint32_t loff1 = (uint32_t)(lrow * p.K + (((lane & 7) ^ lrow ^ 1) << 4));
  const uint8_t* pbase = p.P + (int64_t)i0 * p.K;
  const uint8_t* qbase = p.Q + (int64_t)j0 * p.K;
  auto slab = [&](const uint8_t* base, int n, int rows, int kb, uint32_t ldst) {
    if (!CLAMP) {
      dma16(base + (int64_t)(8 * n) * p.K + kb * 128, (n & 1) ? loff1 : loff0, ldst);
    } else {
      const int row = min(8 * n + lrow, rows - 1);
      dma16(base + kb * 128, (uint32_t)row * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ lrow ^ (n & 1)) << 4), ldst);
    }
  };
  auto p_slab = [&](int r, int kb, int st) {
    slab(pbase, wave * P_INSTR + r, prows, kb, tiles_lds + st * C::TILE_BYTES + (wave * P_INSTR + r) * 1024);
  };
  auto q_slab = [&](int r, int kb, int st) {
    slab(qbase, wave * Q_INSTR + r, qrows, kb,
         tiles_lds + st * C::TILE_BYTES + C::BI * 128 + (wave * Q_INSTR + r) * 1024);
  };

  // ---- L2 prefetch: each lane touches the 128-byte segment of one tile row
  //      for K step kb (P rows then Q rows, one row per lane), so that the LDS
  //      copies of that step, issued a step later, hit in L2. The 4-byte copy
  //      lands in pf_sink. ----
  const bool pf_p = wave * 64 < C::BI;                        // wavefront-uniform
  const uint8_t* pf_base = pf_p ? pbase + (int64_t)(CLAMP ? 0 : wave * 64) * p.K
                                : qbase + (int64_t)(CLAMP ? 0 : wave * 64 - C::BI) * p.K;
  const uint32_t pf_off = CLAMP ? (uint32_t)(pf_p ? min(wave * 64 + lane, prows - 1) : min(wave * 64 - C::BI + lane, qrows - 1)) * (uint32_t)p.K
                                : (uint32_t)lane * (uint32_t)p.K;
  // (the sink address is wavefront-uniform; readfirstlane keeps it in the
  // scalar register the copy's M0 needs)
  auto prefetch = [&](int kb) {
    dma4(pf_base + kb * 128, pf_off, (uint32_t)__builtin_amdgcn_readfirstlane((int)(sink_lds + wave * 256)));
  };

  // ---- scales. The per-row scales (Q rows, then for WGrad the P rows) go to
  //      LDS as [row][4]: 4 consecutive K steps of each row, a group of 4
  //      steps ahead. When K/128 is a multiple of 4, lane t < ROWSC fetches
  //      row t's group with one 16-byte copy; otherwise a row's group is not
  //      16-byte aligned, and four 4-byte copies per wavefront fill the same
  //      layout, lane L taking step L % 4 of row L / 4 of each quarter of the
  //      wavefront's 64 rows (steps past the last repeat it and are never
  //      read). Both are LDS DMA copies, waited for with the operand copies
  //      (plain loads here made the wavefront wait for them, and with them
  //      for every copy in flight, once per group: 7-10 % slower). The last
  //      wavefront's first lanes fetch the block P scales each K step. ----
  auto load_row_scales = [&](int grp) {   // K steps 4grp .. 4grp+3 into rowsc[grp & 1]
#pragma unroll
    for (int pass = 0; pass < C::ROW_PASSES; ++pass) {
      const int r = tid + pass * C::NT;                   // scale row owned by this lane
      const int rw = wave * 64 + pass * C::NT;            // first row of this wavefront (uniform)
      if (rw >= C::ROWSC) continue;
      const bool q_rows = rw < C::BJ;                     // the 64 rows are all Q or all P rows
      const float* rbase = q_rows ? p.Qs + (int64_t)j0 * p.Kb : p.Ps + (int64_t)i0 * p.Kb;
      const int k0 = 4 * grp;
      const uint32_t dst = rowsc_lds + ((grp & 1) * C::ROWSC + rw) * 16;
      if (V4) {
        // Launches of this form always have K/128 a multiple of 4; the
        // runtime test and the plain stores behind it are never taken, but
        // without them the compiler allocates the large row-scaled tile
        // differently and the grouped WGrad ran 2-2.5 % slower (same bits).
        const int rrow = q_rows ? min(r, qrows - 1) : min(r - C::BJ, prows - 1);
        if ((p.Kb & 3) == 0) {
          dma16(rbase, (uint32_t)((rrow * p.Kb + k0) * 4), dst);
        } else {
          const float* src = rbase + (int64_t)rrow * p.Kb;
#pragma unroll
          for (int q = 0; q < 4; ++q) rowsc[grp & 1][r * 4 + q] = k0 + q < p.Kb ? src[k0 + q] : 0.0f;
        }
      } else {
        // (the lane index passes through an empty asm so that the offsets are
        // computed here, once per group, instead of held in registers across
        // the K loop, where the large tile has none to spare)
        int l = lane;
        asm volatile("" : "+v"(l));
        const int kq = min(k0 + (l & 3), p.Kb - 1);
        const int r0 = (q_rows ? rw : rw - C::BJ) + (l >> 2);      // Q or P row of quarter 0
        const int rmax = (q_rows ? qrows : prows) - 1;
#pragma unroll
        for (int qtr = 0; qtr < 4; ++qtr) {
          // Without CLAMP every configuration runs only on whole tiles, so all
          // 64 rows exist and the quarter moves the scalar base, not the lane offset.
          if (CLAMP)
            dma4(rbase, (uint32_t)((min(r0 + 16 * qtr, rmax) * p.Kb + kq) * 4), dst + qtr * 256);
          else
            dma4(rbase + (int64_t)(16 * qtr) * p.Kb, (uint32_t)((r0 * p.Kb + kq) * 4), dst + qtr * 256);
        }
      }
    }
  };
  const int blk_lane = tid - (C::NT - 64);
  const bool bl = !PS_ROW && blk_lane >= 0 && blk_lane < C::BLKSC;
  const int bblk = min((i0 / 128) + max(blk_lane, 0), p.I / 128 - 1);
  auto load_blk_scales = [&](int kb, int st) {
    if (bl) dma4(p.Ps, (uint32_t)((bblk * p.ps_ib + kb * p.ps_kb) * 4), blksc_lds + st * C::BLKSC_PAD * 4);
  };

  f32x4 acc[SI][SJ];
#pragma unroll
  for (int a = 0; a < SI; ++a)
#pragma unroll
    for (int b = 0; b < SJ; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Prologue: scales, then the first NST-1 stages (oldest first).
  constexpr int SLABS = P_INSTR + Q_INSTR;   // copies per wavefront per stage
  load_row_scales(0);
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0) load_blk_scales(min(s0, p.Kb - 1), s0);
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0) {
#pragma unroll
    for (int r = 0; r < P_INSTR; ++r) p_slab(r, min(s0, p.Kb - 1), s0);
#pragma unroll
    for (int r = 0; r < Q_INSTR; ++r) q_slab(r, min(s0, p.Kb - 1), s0);
  }
  wait_dma_keep<(NST - 2) * SLABS>();        // stage 0 (and every scale) has landed
  __syncthreads();

  // ---- main loop. Software pipeline over the SI row slices of the
  //      wavefront tile: the MFMA of (slice a, column slice b) is issued right
  //      before the FMAs that promote (slice a-1, column slice b), so the VALU
  //      promotion of one slice runs while the matrix core works on the next.
  //      The last slice of a K step is promoted at the start of the next K
  //      step (at the first step the carried partials and scales are zero). ----
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  auto load_frag = [&](const uint8_t* t, int row) -> i32x8 {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(t + swz(row, 2 * g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(t + swz(row, 2 * g + 1));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // promote one 16x16 partial: acc += d * (row scale) * (column scale)
  auto promote1 = [&](f32x4& accv, const f32x4& d, float cs, const f32x4& rs) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (PS_ROW)
        accv[r] = __builtin_fmaf(d[r], rs[r] * cs, accv[r]);
      else
        accv[r] = __builtin_fmaf(d[r], cs, accv[r]);
    }
  };
  constexpr int PROMOTE_VALU = PS_ROW ? 8 : 4;
  // Block-scaled roles carry the last slice's promotion into the next K step;
  // the row-scaled role (twice the promotion VALU and registers) promotes it
  // at the end of its own step.
  constexpr bool CARRY = !PS_ROW;

  f32x4 dprev[SJ];
  float ccarry[SJ];
#pragma unroll
  for (int b = 0; b < SJ; ++b) {
    dprev[b] = zero;
    ccarry[b] = 0.0f;
  }
  f32x4 rprev = zero;
  // A step's copies go out over two slices. The loop body is instantiated
  // twice: with 8 wavefronts, the second wavefront of each SIMD (waves 4-7)
  // may issue its copies later than the first, so the two do not stall on
  // copy issue at the same moments: two slices later in WGrad (whose slices
  // carry twice the promotion VALU), one in the medium tile's forward and
  // DGrad, none in the large tile's. Against four slices and a one-slice
  // offset for every role (outputs identical): the grouped WGrad of the 32B
  // linears at 32768 tokens 2-3 % faster, their forward and DGrad 1-2 %. The
  // offset is a compile-time constant so the unrolled slices stay free of
  // branches.
  constexpr int LOAD_SLICES_ = 2;   // slices over which a step's copies are spread
  auto main_loop = [&](auto copy_offset) {
  constexpr int OFF = decltype(copy_offset)::value;
  // one K step; COPIES false: the step sends no copies (the last step of a
  // two-stage tile, whose next stage would never be read)
  auto kstep = [&](const int kb, auto copies) {
    constexpr bool COPIES = decltype(copies)::value;
    const int st = kb % NST;        // stage of step kb
    const uint8_t* tp = tiles[st];
    const uint8_t* tq = tiles[st] + C::BI * 128;
    const float* rsc = &rowsc[(kb >> 2) & 1][kb & 3];   // scale of row r at rsc[4 r]

    // First P fragment, then the Q fragments in the order the first slice
    // uses them, so its first MFMA waits for two fragments only. The P
    // fragments run PF_DEPTH slices ahead of their MFMAs (a ring of
    // PF_DEPTH + 1), which hides the LDS latency of a slice behind the MFMAs
    // of the PF_DEPTH slices before it.
    constexpr int PF_DEPTH = 2;
    i32x8 pring[PF_DEPTH + 1];
    pring[0] = load_frag(tp, wi * C::WI + r16);
    i32x8 qf[SJ];
    float cj[SJ];
#pragma unroll
    for (int b = 0; b < SJ; ++b) {
      const int row = wj * C::WJ + b * 16 + r16;
      qf[b] = load_frag(tq, row);
      cj[b] = rsc[4 * row];
    }
    if (!PS_ROW) {
      const float psw = blksc[st][(wi * C::WI) / 128];
#pragma unroll
      for (int b = 0; b < SJ; ++b) cj[b] *= psw;
    }
#pragma unroll
    for (int a = 1; a < PF_DEPTH; ++a) pring[a] = load_frag(tp, wi * C::WI + a * 16 + r16);
    // the next group of row scales goes out at the first step of each group
    if ((kb & 3) == 0 && kb + 4 < p.Kb) load_row_scales((kb >> 2) + 1);

    // The next stage's tiles go out spread over the first slices (a few
    // copies at a time keep the memory pipeline from stalling the wavefront);
    // with three or four stages the last steps re-fetch the last K step into
    // the idle buffer (never read; it keeps every step's copy count).
    const int kn = min(kb + NST - 1, p.Kb - 1);
    const int sn = st == 0 ? NST - 1 : st - 1;    // stage of step kb + NST - 1 (idle now)
    if (COPIES) load_blk_scales(kn, sn);
    constexpr int LOAD_SLICES = LOAD_SLICES_;
    static_assert(P_INSTR % LOAD_SLICES == 0 && Q_INSTR % LOAD_SLICES == 0 && SI >= LOAD_SLICES + OFF, "load spread");
#pragma unroll
    for (int a = 0; a < SI; ++a) {
      if (COPIES && a >= OFF && a < OFF + LOAD_SLICES) {
        const int al = a - OFF;
#pragma unroll
        for (int r = 0; r < P_INSTR / LOAD_SLICES; ++r) p_slab(al * (P_INSTR / LOAD_SLICES) + r, kn, sn);
#pragma unroll
        for (int r = 0; r < Q_INSTR / LOAD_SLICES; ++r) q_slab(al * (Q_INSTR / LOAD_SLICES) + r, kn, sn);
      }
      if (a + PF_DEPTH < SI)
        pring[(a + PF_DEPTH) % (PF_DEPTH + 1)] = load_frag(tp, wi * C::WI + (a + PF_DEPTH) * 16 + r16);
      const i32x8 pf = pring[a % (PF_DEPTH + 1)];
      f32x4 rs = zero;
      if (PS_ROW) {
        const int prow = C::BJ + wi * C::WI + a * 16 + 4 * g;
        rs = f32x4{rsc[4 * prow], rsc[4 * prow + 4], rsc[4 * prow + 8], rsc[4 * prow + 12]};
      }
#pragma unroll
      for (int b = 0; b < SJ; ++b) {
        const f32x4 dcur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf, qf[b], zero, 0, 0, 0, 0, 0, 0);
        if (a > 0)
          promote1(acc[a - 1][b], dprev[b], cj[b], rprev);
        else if (CARRY)
          promote1(acc[SI - 1][b], dprev[b], ccarry[b], rprev);
        dprev[b] = dcur;
      }
      // MFMAs, then the promotions of the partials they replaced, in turn:
      // two at a time on the large tile (1-2 % faster there than one at a
      // time, 1-3 % slower on the medium tile), one at a time otherwise (the
      // row-scaled role schedules better left to the compiler)
      if (!PS_ROW) {
        constexpr int SG = C::BJ == 256 ? 2 : 1;
        static_assert(SJ % SG == 0, "schedule groups of SG column slices");
#pragma unroll
        for (int b = 0; b < SJ; b += SG) {
          __builtin_amdgcn_sched_group_barrier(0x008, SG, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, SG * PROMOTE_VALU, 0);
        }
      }
      rprev = rs;
    }
    if (CARRY) {
#pragma unroll
      for (int b = 0; b < SJ; ++b) ccarry[b] = cj[b];
    } else {
#pragma unroll
      for (int b = 0; b < SJ; ++b) promote1(acc[SI - 1][b], dprev[b], cj[b], rprev);
    }

    // the copies for step kb+1 (issued NST-2 steps ago) have landed; this
    // step's copies may stay in flight when NST > 2
    if (PF_L2) prefetch(min(kb + NST, p.Kb - 1));
    wait_dma_keep<(NST - 2) * SLABS + (PF_L2 ? 1 : 0)>();
    __syncthreads();
  };
  // With two stages each step waits for all its copies, so the last step
  // sends none (it used to re-fetch the last K step into the idle buffer,
  // never read: a third of all copies at two K steps per tile; 256-token
  // grouped WGrad 2.4 %, 32768-token forward 0.9 % faster); with more
  // stages every step sends its share, so that the wait counts hold.
  if (NST == 2) {
    for (int kb = 0; kb + 1 < p.Kb; ++kb) kstep(kb, std::true_type{});
    kstep(p.Kb - 1, std::false_type{});
  } else {
    for (int kb = 0; kb < p.Kb; ++kb) kstep(kb, std::true_type{});
  }
  };

  constexpr int OFF_HI = C::NT != 512                        ? 0
                         : (PS_ROW && SI >= LOAD_SLICES_ + 2) ? 2
                         : C::BJ == 256                       ? 0
                         : (SI >= LOAD_SLICES_ + 1)           ? 1
                                                              : 0;
  if (OFF_HI && wave >= 4)
    main_loop(std::integral_constant<int, OFF_HI>{});
  else
    main_loop(std::integral_constant<int, 0>{});
  if (CARRY) {
#pragma unroll
    for (int b = 0; b < SJ; ++b) promote1(acc[SI - 1][b], dprev[b], ccarry[b], rprev);
  }
  wait_dma_keep<0>();   // no copy into LDS may outlive the workgroup

  // ---- epilogue. Lane holds out[j][i .. i+3] for each (a, b). The wavefront
  //      writes its WJ x WI bf16 block into LDS (the stage buffers are free
  //      once every wavefront has left the loop), rows of WI*2 bytes with the
  //      16-byte chunk index XOR-swizzled by the row, then stores whole
  //      16-byte chunks, 2*WI contiguous bytes per output row (storing the
  //      8-byte pieces straight from registers touched 16 rows per
  //      instruction; this is 2-5 % faster at large K and 1.45x faster where
  //      the output dominates, e.g. a 256-token WGrad). ----
  {
    constexpr int ROWB = C::WI * 2;               // bytes per row of the wavefront block
    constexpr int CHUNKS = ROWB / 16;             // 16-byte chunks per row
    static_assert((CHUNKS & (CHUNKS - 1)) == 0 && C::WJ * ROWB * (C::NT / 64) <= NST * C::TILE_BYTES,
                  "epilogue staging fits the stage buffers");
    uint8_t* eb = &tiles[0][0] + wave * (C::WJ * ROWB);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < SI; ++a) {
#pragma unroll
      for (int b = 0; b < SJ; ++b) {
        const int jr = b * 16 + r16;
        const int byte = a * 32 + 8 * g;          // of row jr
        const int ch = (byte >> 4) ^ (jr & (CHUNKS - 1));
        *reinterpret_cast<u32x2*>(eb + jr * ROWB + ch * 16 + (byte & 15)) =
            u32x2{pack_bf16x2(acc[a][b][0], acc[a][b][1]), pack_bf16x2(acc[a][b][2], acc[a][b][3])};
      }
    }
    constexpr int ROWS_PER_PASS = 64 / CHUNKS;
    const int c = lane % CHUNKS;
    const int i = i0 + wi * C::WI + c * 8;
#pragma unroll
    for (int k = 0; k < C::WJ / ROWS_PER_PASS; ++k) {
      const int jr = lane / CHUNKS + ROWS_PER_PASS * k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(eb + jr * ROWB + ((c ^ (jr & (CHUNKS - 1))) * 16));
      const int j = j0 + wj * C::WJ + jr;
      // Iout is a multiple of 8, so each 16-byte chunk is stored whole or not
      // at all. Non-temporal: the output is not read again by this kernel, and
      // keeping it out of L2 leaves room for the operand bands that other
      // tiles still read (1-2.5 % faster on the large GEMMs, 7-9 % on a
      // 256-token grouped WGrad, whose time is its output).
      if ((!CLAMP || j < p.J) && i < p.Iout)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.out + (int64_t)j * p.ldo + i));
    }
  }
#endif
}

template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST, bool CLAMP>
__global__ __launch_bounds__(64 * WAVES_I * WAVES_J) void fp8_gemm_kernel(GemmParams p) {
  gemm_body<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP, true>(p, (int)blockIdx.x, (int)gridDim.x);
}

// Several problems of one role in one launch: problem g owns the blocks
// [start[g], start[g+1]); each problem's range starts at a multiple of the XCD
// count so that its blocks keep the XCD-aware order of a plain launch (the
// blocks of the padding exit at once).
constexpr int kMaxGroup = 16;
struct GroupedParams {
  int count;
  int start[kMaxGroup + 1];
  GemmParams prob[kMaxGroup];
};

template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST, bool CLAMP>
__global__ __launch_bounds__(64 * WAVES_I * WAVES_J) void fp8_gemm_grouped_kernel(GroupedParams gp) {
  const int bid = (int)blockIdx.x;
  const int g = grouped_problem(bid, gp.start, gp.count);   // uniform over the workgroup
  const GemmParams& p = gp.prob[g];
  const int nblk = p.tiles_i * p.tiles_j;
  const int local = bid - gp.start[g];
  if (local >= nblk) return;
  gemm_body<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP, true>(p, local, nblk);
}
// The same where some problem's K/128 is not a multiple of 4 (plain calls
// of such a K go out as a group of one): a kernel of its own, so that the
// other form of the scale copies costs the common one no registers (in the
// plain kernel it made the large tile spill). (Both are written out in full:
// the grouped WGrad measured 4 % slower with their common part in a shared
// inline function, whose extra level changed the register allocation.)
template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST, bool CLAMP>
__global__ __launch_bounds__(64 * WAVES_I * WAVES_J) void fp8_gemm_grouped_kernel_unaligned(GroupedParams gp) {
  const int bid = (int)blockIdx.x;
  const int g = grouped_problem(bid, gp.start, gp.count);   // uniform over the workgroup
  const GemmParams& p = gp.prob[g];
  const int nblk = p.tiles_i * p.tiles_j;
  const int local = bid - gp.start[g];
  if (local >= nblk) return;
  gemm_body<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP, false>(p, local, nblk);
}

// ----------------------------------------------------------------------------
// Launch one tile configuration.
// ----------------------------------------------------------------------------
template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST, bool CLAMP>
static hipError_t run_grouped_cfg(const GemmParams* probs, int count, hipStream_t stream) {
  using C = GemmCfg<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST>;
  GroupedParams gp{};
  gp.count = count;
  // Each problem's block range starts at a multiple of the XCD count; with
  // 8 wavefronts (one workgroup per compute unit) at a multiple of 256, so
  // that a problem's chip-wide 16 x 16 supertiles line up with the rounds of
  // 256 workgroups the chip runs at once (grouped WGrad of the 32B linears at
  // 32768 tokens: 12.07 -> 11.99 ms; the padding blocks exit at once).
  constexpr int ALIGN = C::NT == 512 ? 256 : NUM_XCD;
  int tiles[kMaxGroup];
  bool v4 = true;
  for (int g = 0; g < count; ++g) {
    GemmParams q = probs[g];
    v4 = v4 && (q.Kb & 3) == 0;
    q.tiles_i = (q.I + C::BI - 1) / C::BI;
    q.tiles_j = (q.J + C::BJ - 1) / C::BJ;
    gp.prob[g] = q;
    tiles[g] = q.tiles_i * q.tiles_j;
  }
  const int total = grouped_layout(tiles, count, ALIGN, gp.start);
  if (v4)
    hipLaunchKernelGGL((fp8_gemm_grouped_kernel<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP>), dim3(total),
                       dim3(C::NT), 0, stream, gp);
  else
    hipLaunchKernelGGL((fp8_gemm_grouped_kernel_unaligned<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP>),
                       dim3(total), dim3(C::NT), 0, stream, gp);
  return hipGetLastError();
}

template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW, int NST, bool CLAMP>
static hipError_t run_gemm_cfg(GemmParams p, hipStream_t stream) {
  using C = GemmCfg<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST>;
  // a K/128 that is not a multiple of 4: the grouped kernel with that form of
  // the scale copies, one problem (same tiles, same order, same bits)
  if ((p.Kb & 3) != 0) return run_grouped_cfg<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP>(&p, 1, stream);
  p.tiles_i = (p.I + C::BI - 1) / C::BI;
  p.tiles_j = (p.J + C::BJ - 1) / C::BJ;
  const int nblk = p.tiles_i * p.tiles_j;
  hipLaunchKernelGGL((fp8_gemm_kernel<WAVES_I, WAVES_J, SI, SJ, PS_ROW, NST, CLAMP>), dim3(nblk), dim3(C::NT), 0,
                     stream, p);
  return hipGetLastError();
}

// Four tile configurations. Every one reduces K in the same order (one MFMA
// and one promotion per 128-long block, in order), so the choice changes no
// output bit.
//  large: 256 x 256 tile, 8 wavefronts (2 per SIMD) of 128 x 64, 2 LDS
//         stages. (A 256 x 128 tile with one wavefront per SIMD and 3 stages
//         measured slower: one wavefront cannot hide its own LDS latency.)
//  small: 128 x 64 tile, 4 wavefronts of 64 x 32, 3 LDS stages (two
//         workgroups per compute unit): for problems with fewer large tiles
//         than compute units (decode-sized M, small outputs), where it
//         measured 1.1-2.5x faster; more workgroups and a deeper prefetch.
//  tiny:  64 x 64 tile, 4 wavefronts of 32 x 32, 4 LDS stages (67 KB, two
//         workgroups per compute unit): when even the small tiles are too few
//         (under two per compute unit), e.g. decode and the long-contraction
//         linears at 256 tokens, where the extra workgroups measured 10-25 %
//         faster than the small tile. These shapes stream their weights with
//         little reuse; the fourth stage keeps one more K step of copies in
//         flight (with weights rotated past the last-level cache: 3-24 %
//         faster than 3 stages on every decode and 256-token shape measured).
//  medium: 256 x 128 tile, 8 wavefronts of 128 x 32, 3 LDS stages (148-156
//         KB, one workgroup per compute unit): instead of the large tile when
//         the large tiles end just past a whole round of the 256 compute
//         units (320 tiles are 1.25 rounds: the last round leaves 3/4 of the
//         chip idle). Per FLOP it measured 4-9 % slower than the large tile;
//         it is chosen when rounds x cost per tile is lower, with a medium
//         tile costing 0.54 of a large one (measured on the linears of a
//         32B-parameter model at 4096 tokens: 11-16 % faster where the large
//         tiles number 320, slower at 400, 448 and 1728).
// The large and medium ones run only where both output dimensions hold a
// whole tile, so only the tiny one has a clamped-row (CLAMP) instantiation.
constexpr int64_t kComputeUnits = 256;
template <bool PS_ROW>
static hipError_t run_gemm(GemmParams p, hipStream_t stream) {
  const int64_t large_tiles = (int64_t)((p.I + 255) / 256) * ((p.J + 255) / 256);
  if (p.I >= 256 && p.J >= 256 && large_tiles >= kComputeUnits) {
    const int64_t medium_tiles = (int64_t)((p.I + 255) / 256) * ((p.J + 127) / 128);
    const int64_t large_rounds = (large_tiles + kComputeUnits - 1) / kComputeUnits;
    const int64_t medium_rounds = (medium_tiles + kComputeUnits - 1) / kComputeUnits;
    if (54 * medium_rounds < 100 * large_rounds) return run_gemm_cfg<2, 4, 8, 2, PS_ROW, 3, false>(p, stream);
    return run_gemm_cfg<2, 4, 8, 4, PS_ROW, 2, false>(p, stream);
  }
  // A few hundred tokens against a wide weight (the GEMM is HBM-bound): when
  // the medium tiles make one round of at least 3/4 of the compute units, each
  // workgroup streams its own 256 weight rows once, where the small tiles'
  // four workgroups per 128-row weight band share it through L2 (measured
  // 30 % faster at 256 tokens for 27648 weight rows; with fewer tiles the
  // chip is left idle and the small and tiny tiles win).
  const int64_t medium_tiles = (int64_t)((p.I + 255) / 256) * ((p.J + 127) / 128);
  if (p.I >= 256 && p.J >= 128 && p.J <= 256 && 4 * medium_tiles >= 3 * kComputeUnits &&
      medium_tiles <= kComputeUnits)
    return run_gemm_cfg<2, 4, 8, 2, PS_ROW, 3, false>(p, stream);
  const int64_t small_tiles = (int64_t)((p.I + 127) / 128) * ((p.J + 63) / 64);
  if (p.I >= 128 && p.J >= 64 && small_tiles >= 512) return run_gemm_cfg<2, 2, 4, 2, PS_ROW, 3, false>(p, stream);
  if (p.I >= 64 && p.J >= 64) return run_gemm_cfg<2, 2, 2, 2, PS_ROW, 4, false>(p, stream);
  return run_gemm_cfg<2, 2, 2, 2, PS_ROW, 4, true>(p, stream);
}

// One configuration for the whole group: the large one when every problem
// qualifies for it and the group fills the chip, else the small one (with
// clamped rows when some problem is smaller than one small tile).
template <bool PS_ROW>
static hipError_t run_grouped(const GemmParams* probs, int count, hipStream_t stream) {
  bool large_ok = true, small_ok = true;
  int64_t large_tiles = 0;
  for (int g = 0; g < count; ++g) {
    const GemmParams& q = probs[g];
    large_ok = large_ok && q.I >= 256 && q.J >= 256;
    small_ok = small_ok && q.I >= 128 && q.J >= 64;
    large_tiles += (int64_t)((q.I + 255) / 256) * ((q.J + 255) / 256);
  }
  if (large_ok && large_tiles >= 256) return run_grouped_cfg<2, 4, 8, 4, PS_ROW, 2, false>(probs, count, stream);
  if (small_ok) return run_grouped_cfg<2, 2, 4, 2, PS_ROW, 3, false>(probs, count, stream);
  return run_grouped_cfg<2, 2, 4, 2, PS_ROW, 3, true>(probs, count, stream);
}

// Operand roles. All three run D[i][j] = sum_k P[i,k] Q[j,k], written to out[j][i].
// M, N, K are the logical sizes; the code tensors have them rounded up to 128
// along their grouped dimensions.
static int blocks128(int64_t n) { return (int)((n + 127) / 128); }

static GemmParams fwd_params(const GemmProblem& pr) {
  GemmParams p{};
  const int Nb = blocks128(pr.N), Kb = blocks128(pr.K);
  p.P = pr.b; p.Ps = pr.bs; p.Q = pr.a; p.Qs = pr.as; p.out = static_cast<uint16_t*>(pr.out);
  p.I = 128 * Nb; p.J = (int)pr.M; p.K = 128 * Kb; p.Kb = Kb;
  p.Iout = (int)pr.N; p.ldo = (int)pr.N;
  p.ps_ib = Kb;  // ws[n/128][kb]
  p.ps_kb = 1;
  return p;
}

static GemmParams dgrad_params(const GemmProblem& pr) {
  GemmParams p{};
  const int Nb = blocks128(pr.N), Kb = blocks128(pr.K);
  p.P = pr.b; p.Ps = pr.bs; p.Q = pr.a; p.Qs = pr.as; p.out = static_cast<uint16_t*>(pr.out);
  p.I = 128 * Kb; p.J = (int)pr.M; p.K = 128 * Nb; p.Kb = Nb;
  p.Iout = (int)pr.K; p.ldo = (int)pr.K;
  p.ps_ib = 1;   // ws[nb][k/128]: i = k selects the column block
  p.ps_kb = Kb;  //                 the contraction block nb selects the row
  return p;
}

static GemmParams wgrad_params(const GemmProblem& pr) {
  GemmParams p{};
  p.P = pr.b; p.Ps = pr.bs; p.Q = pr.a; p.Qs = pr.as; p.out = static_cast<uint16_t*>(pr.out);
  p.I = (int)pr.K; p.J = (int)pr.N; p.K = (int)pr.M; p.Kb = (int)(pr.M / 128);
  p.Iout = (int)pr.K; p.ldo = (int)pr.K;
  return p;
}

hipError_t launch_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                           void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return run_gemm<false>(fwd_params(GemmProblem{xq, xs, wq, ws, y, M, N, K}), stream);
}

hipError_t launch_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                             const float* ws, void* dx, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream) {
  return run_gemm<false>(dgrad_params(GemmProblem{dyq, dys, wq_t, ws, dx, M, N, K}), stream);
}

hipError_t launch_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t,
                             const float* xs_t, void* dw, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream) {
  return run_gemm<true>(wgrad_params(GemmProblem{dyq_t, dys_t, xq_t, xs_t, dw, M, N, K}), stream);
}

hipError_t launch_gemm_grouped(GemmRole role, const GemmProblem* problems, int count, hipStream_t stream) {
  for (int g0 = 0; g0 < count; g0 += kMaxGroup) {
    const int n = count - g0 < kMaxGroup ? count - g0 : kMaxGroup;
    GemmParams ps[kMaxGroup];
    for (int g = 0; g < n; ++g) {
      const GemmProblem& pr = problems[g0 + g];
      ps[g] = role == GemmRole::Fwd ? fwd_params(pr) : role == GemmRole::Dgrad ? dgrad_params(pr) : wgrad_params(pr);
    }
    const hipError_t e = role == GemmRole::Wgrad ? run_grouped<true>(ps, n, stream) : run_grouped<false>(ps, n, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp8bsq
