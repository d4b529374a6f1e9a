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
// and writes out as a row-major [J, I] bf16 matrix.
//   forward: P = Wq [N, K] (block scales), Q = Xq [M, K]   -> out = Y  [M, N]
//   DGrad  : P = Wq^T [K, N] (block scales, read transposed), Q = dYq [M, N] -> dX [M, K]
//   WGrad  : P = Xq^T [K, M] (row scales), Q = dYq^T [N, M] -> dW [N, K]
//
// Each 128-long K block is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16
// output tile, so the block's partial sum comes out of a single MFMA with a
// zero accumulator and is promoted into the fp32 running sum with one FMA per
// element: acc += partial * ps * qs. In the MFMA result layout a lane holds
// four consecutive i of one j, so the Q scale is one value per lane and a
// block P scale is uniform over the wavefront.
//
// Tiles: a workgroup owns a BI x BJ output tile and walks K in 128-byte steps.
// Both operand tiles of a step are staged in LDS (double-buffered) with their
// 16-byte chunks XOR-swizzled by row so that the MFMA fragment reads are free
// of bank conflicts. Workgroups are mapped to tiles so that each XCD works on
// a compact band of the output (its own L2), in groups along i.
#include "device_common.h"
#include "launch.h"

namespace fp8bsq {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct GemmParams {
  const uint8_t* P;
  const float* Ps;
  const uint8_t* Q;
  const float* Qs;
  uint16_t* out;
  int I, J, K, Kb;
  int ps_ib, ps_kb;  // block P scale of (i, kb) at Ps[(i / 128) * ps_ib + kb * ps_kb]
  int tiles_i, tiles_j;
};

// XCD-aware tile order. The hardware hands out workgroup ids round-robin over
// the 8 XCDs; ids b, b+8, b+16, ... share an XCD. Renumber so that each XCD
// gets a contiguous range of logical tiles, then walk logical tiles in groups
// of GROUP_I tiles along i (all j for one group before the next group).
constexpr int NUM_XCD = 8;
constexpr int GROUP_I = 8;

__device__ __forceinline__ void map_tile(int bid, int nblk, int tiles_i, int tiles_j, int& ti, int& tj) {
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

template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW>
struct GemmCfg {
  static constexpr int WI = SI * 16, WJ = SJ * 16;              // wavefront tile
  static constexpr int BI = WAVES_I * WI, BJ = WAVES_J * WJ;    // workgroup tile
  static constexpr int NT = 64 * WAVES_I * WAVES_J;
  static constexpr int P_LOADS = BI * 8 / NT;                    // 16-byte loads per thread
  static constexpr int Q_LOADS = BJ * 8 / NT;
  static constexpr int PS_COUNT = PS_ROW ? BI : BI / 128;        // P scales per K step
  static constexpr int TILE_BYTES = (BI + BJ) * 128;
  static constexpr int SCALE_FLOATS = BJ + PS_COUNT;
  static_assert(BI * 8 % NT == 0 && BJ * 8 % NT == 0, "loads must divide evenly");
  static_assert(NT >= BJ + PS_COUNT, "one scale load per thread at most");
  static_assert(PS_ROW || (128 % WI == 0), "a block-scaled wavefront must sit inside one 128-row block");
  static_assert(BI % 128 == 0, "BI must be a multiple of 128");
};

// Byte offset of 16-byte chunk `chunk` of tile row `row` (rows are 128 bytes).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int WAVES_I, int WAVES_J, int SI, int SJ, bool PS_ROW>
__global__ __launch_bounds__(64 * WAVES_I * WAVES_J) void fp8_gemm_kernel(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses LDS address-space casts, device pass only
  using C = GemmCfg<WAVES_I, WAVES_J, SI, SJ, PS_ROW>;
  __shared__ __align__(16) uint8_t tiles[2][C::TILE_BYTES];
  __shared__ __align__(16) float scales[2][C::SCALE_FLOATS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wi = wave % WAVES_I, wj = wave / WAVES_I;
  const int g = lane >> 4, r16 = lane & 15;

  int ti, tj;
  map_tile(blockIdx.x, gridDim.x, p.tiles_i, p.tiles_j, ti, tj);
  const int i0 = ti * C::BI, j0 = tj * C::BJ;

  // ---- global -> LDS loads. Each wavefront instruction moves 64 x 16 bytes
  //      straight into 1 KB of LDS (8 tile rows), lane L landing at byte 16L.
  //      Lane L therefore fetches the global chunk that the swizzled layout
  //      keeps at that spot: row 8n + L/8, logical chunk (L%8) ^ (L/8).
  //      Rows past the end are clamped into range; they feed only outputs
  //      that are never stored. ----
  constexpr int P_INSTR = C::BI / 8 / (C::NT / 64);   // 1 KB instructions per wavefront
  constexpr int Q_INSTR = C::BJ / 8 / (C::NT / 64);
  static_assert(P_INSTR * 8 * (C::NT / 64) == C::BI && Q_INSTR * 8 * (C::NT / 64) == C::BJ, "tile rows per wave");
  const int lrow = lane >> 3;                        // row within the 8-row slab
  const int lchunk = (lane & 7) ^ lrow;              // logical chunk fetched by this lane
  const uint8_t* pbase = p.P + (int64_t)i0 * p.K;
  const uint8_t* qbase = p.Q + (int64_t)j0 * p.K;
  uint32_t poff[P_INSTR], qoff[Q_INSTR];
#pragma unroll
  for (int r = 0; r < P_INSTR; ++r) {
    const int row = 8 * (wave * P_INSTR + r) + lrow;
    poff[r] = (uint32_t)(min(row, p.I - 1 - i0) * p.K + lchunk * 16);
  }
#pragma unroll
  for (int r = 0; r < Q_INSTR; ++r) {
    const int row = 8 * (wave * Q_INSTR + r) + lrow;
    qoff[r] = (uint32_t)(min(row, p.J - 1 - j0) * p.K + lchunk * 16);
  }
  // Scales: lanes of wavefronts 0.. fetch one float each into scales[st][0 .. SCALE_FLOATS).
  const float* sg = nullptr;
  int s_step = 0;
  if (tid < C::BJ) {
    sg = p.Qs + (int64_t)min(j0 + tid, p.J - 1) * p.Kb;
    s_step = 1;
  } else if (tid < C::BJ + C::PS_COUNT) {
    const int k = tid - C::BJ;
    if (PS_ROW) {
      sg = p.Ps + (int64_t)min(i0 + k, p.I - 1) * p.Kb;
      s_step = 1;
    } else {
      sg = p.Ps + (int64_t)min((i0 / 128) + k, p.I / 128 - 1) * p.ps_ib;
      s_step = p.ps_kb;
    }
  }
  auto issue_loads = [&](int kb, int st) {
    typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
    for (int r = 0; r < P_INSTR; ++r)
      __builtin_amdgcn_global_load_lds(pbase + poff[r] + kb * 128,
                                       (lds_void*)(&tiles[st][(wave * P_INSTR + r) * 1024]), 16, 0, 0);
#pragma unroll
    for (int r = 0; r < Q_INSTR; ++r)
      __builtin_amdgcn_global_load_lds(qbase + qoff[r] + kb * 128,
                                       (lds_void*)(&tiles[st][C::BI * 128 + (wave * Q_INSTR + r) * 1024]), 16, 0, 0);
    if (sg) __builtin_amdgcn_global_load_lds(sg + (int64_t)kb * s_step, (lds_void*)(&scales[st][wave * 64]), 4, 0, 0);
  };

  f32x4 acc[SI][SJ];
#pragma unroll
  for (int a = 0; a < SI; ++a)
#pragma unroll
    for (int b = 0; b < SJ; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  issue_loads(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = 0; kb < p.Kb; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < p.Kb) issue_loads(kb + 1, st ^ 1);

    const uint8_t* tp = tiles[st];
    const uint8_t* tq = tiles[st] + C::BI * 128;
    const float* sq = scales[st];
    const float* sp = scales[st] + C::BJ;

    i32x8 qf[SJ];
    float qsc[SJ];
#pragma unroll
    for (int b = 0; b < SJ; ++b) {
      const int row = wj * C::WJ + b * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(tq + swz(row, 2 * g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(tq + swz(row, 2 * g + 1));
      qf[b] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      qsc[b] = sq[row];
    }
    float cj[SJ];
    if (!PS_ROW) {
      const float psw = sp[(wi * C::WI) / 128];
#pragma unroll
      for (int b = 0; b < SJ; ++b) cj[b] = qsc[b] * psw;
    }

#pragma unroll
    for (int a = 0; a < SI; ++a) {
      const int row = wi * C::WI + a * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(tp + swz(row, 2 * g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(tp + swz(row, 2 * g + 1));
      const i32x8 pf = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      f32x4 ps4;
      if (PS_ROW) ps4 = *reinterpret_cast<const f32x4*>(sp + wi * C::WI + a * 16 + 4 * g);
#pragma unroll
      for (int b = 0; b < SJ; ++b) {
        const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf, qf[b], zero, 0, 0, 0, 0, 0, 0);
        if (PS_ROW) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[a][b][r] = __builtin_fmaf(d[r], ps4[r] * qsc[b], acc[a][b][r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[a][b][r] = __builtin_fmaf(d[r], cj[b], acc[a][b][r]);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads into the other stage have landed
    __syncthreads();
  }

  // ---- epilogue: lane holds out[j][i .. i+3] for each (a, b) ----
#pragma unroll
  for (int a = 0; a < SI; ++a) {
    const int i = i0 + wi * C::WI + a * 16 + 4 * g;
#pragma unroll
    for (int b = 0; b < SJ; ++b) {
      const int j = j0 + wj * C::WJ + b * 16 + r16;
      if (j < p.J && i < p.I) {
        const u32x2 v = u32x2{pack_bf16x2(acc[a][b][0], acc[a][b][1]), pack_bf16x2(acc[a][b][2], acc[a][b][3])};
        *reinterpret_cast<u32x2*>(p.out + (int64_t)j * p.I + i) = v;
      }
    }
  }
#endif
}

// ----------------------------------------------------------------------------
// Tile configurations. The large one keeps two wavefronts per SIMD (512
// threads, 256 x 256 output per workgroup, 128 x 64 per wavefront).
// ----------------------------------------------------------------------------
template <bool PS_ROW>
static hipError_t run_gemm(GemmParams p, hipStream_t stream) {
  constexpr int WAVES_I = 2, WAVES_J = 4, SI = 8, SJ = 4;
  using C = GemmCfg<WAVES_I, WAVES_J, SI, SJ, PS_ROW>;
  p.tiles_i = (p.I + C::BI - 1) / C::BI;
  p.tiles_j = (p.J + C::BJ - 1) / C::BJ;
  const int nblk = p.tiles_i * p.tiles_j;
  hipLaunchKernelGGL((fp8_gemm_kernel<WAVES_I, WAVES_J, SI, SJ, PS_ROW>), dim3(nblk), dim3(C::NT), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                           void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  GemmParams p{};
  p.P = wq; p.Ps = ws; p.Q = xq; p.Qs = xs; p.out = static_cast<uint16_t*>(y);
  p.I = (int)N; p.J = (int)M; p.K = (int)K; p.Kb = (int)(K / 128);
  p.ps_ib = (int)(K / 128);  // ws[n/128][kb]
  p.ps_kb = 1;
  return run_gemm<false>(p, stream);
}

hipError_t launch_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq_t,
                             const float* ws, void* dx, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream) {
  GemmParams p{};
  p.P = wq_t; p.Ps = ws; p.Q = dyq; p.Qs = dys; p.out = static_cast<uint16_t*>(dx);
  p.I = (int)K; p.J = (int)M; p.K = (int)N; p.Kb = (int)(N / 128);
  p.ps_ib = 1;               // ws[nb][k/128]: i = k selects the column block
  p.ps_kb = (int)(K / 128);  //                 the contraction block nb selects the row
  return run_gemm<false>(p, stream);
}

hipError_t launch_gemm_wgrad(const uint8_t* dyq_t, const float* dys_t, const uint8_t* xq_t,
                             const float* xs_t, void* dw, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream) {
  GemmParams p{};
  p.P = xq_t; p.Ps = xs_t; p.Q = dyq_t; p.Qs = dys_t; p.out = static_cast<uint16_t*>(dw);
  p.I = (int)K; p.J = (int)N; p.K = (int)M; p.Kb = (int)(M / 128);
  return run_gemm<true>(p, stream);
}

}  // namespace fp8bsq
