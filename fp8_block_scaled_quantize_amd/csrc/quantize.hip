// Quantizer kernels: 1x128 row groups, 128x128 blocks, 128x1 transposed groups.
//
// Source: Resumen Técnico: Jet-RL (gist.science), "Esquema de Cuantización":
// activations in 1x128 groups, weights in 128x128 blocks, WGrad operands in
// 1x128 / 128x1 groups along the tokens, saved activations in FP8.
//
// All three are HBM-bound streaming kernels: every bf16 element is read once
// with 16-byte coalesced loads and every E4M3 byte written once. The group
// amax is reduced inside the wavefront with DPP moves; the 128x1 kernel
// transposes its output tile through LDS so both its reads and its writes
// stay coalesced.
//
// Channel counts that are not a multiple of 128 (any multiple of 8, so bf16
// rows stay 16-byte aligned) end in a partial group. The TAIL instantiation
// of each kernel reads the 16-byte chunks past the last channel as +0 (from a
// clamped, in-bounds address): +0 leaves the amax of the valid elements
// alone and encodes to 0x00, so the code tensors come out padded to whole
// groups with +0 codes (row length Kp = K rounded up to 128). Aligned shapes
// run the instantiation without the masks.
#include "device_common.h"
#include "launch.h"
#include "tile_map.h"

namespace fp8bsq {

// Grid limits the launchers respect: at most kMaxGridY workgroups along y
// and at most kMaxBlocks1D along x of a 1-D grid; larger problems go out as
// several launches, each with its block offset.
constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxBlocks1D = (int64_t)1 << 22;

// ============================================================================
// 1x128: the codes xq [M, Kp] are a flat array of G = M*Kp/128 groups of 128
// bytes and group g's scale is xs[g]. With K % 128 == 0 the input is the same
// flat array of groups; otherwise (TAIL) group g is row g / Kg, group g % Kg
// of the input. Each group is handled by 8 lanes; lane j holds elements
// 8j..8j+7 and 64+8j..64+8j+7, so each load instruction reads 128 contiguous
// bytes per group.
// ============================================================================
constexpr int ACT_THREADS = 256;
constexpr int ACT_PASSES = 2;
constexpr int ACT_GROUPS_PER_PASS = ACT_THREADS / 8;
constexpr int ACT_GROUPS_PER_BLOCK = ACT_GROUPS_PER_PASS * ACT_PASSES;

__device__ __forceinline__ void unpack8(const u32x4& r, float* v) {
  v[0] = bf16_lo(r[0]); v[1] = bf16_hi(r[0]);
  v[2] = bf16_lo(r[1]); v[3] = bf16_hi(r[1]);
  v[4] = bf16_lo(r[2]); v[5] = bf16_hi(r[2]);
  v[6] = bf16_lo(r[3]); v[7] = bf16_hi(r[3]);
}

template <bool TAIL>
__global__ __launch_bounds__(ACT_THREADS) void quant_act_1x128_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, float* __restrict__ xs, int64_t G,
    int64_t blk0, int K, int Kg) {
  const int t = threadIdx.x;
  const int j = t & 7;
  const int64_t blk = blk0 + blockIdx.x;
  u32x4 raw[ACT_PASSES][2];
  int64_t grp[ACT_PASSES];
#pragma unroll
  for (int p = 0; p < ACT_PASSES; ++p) {
    const int64_t g = blk * ACT_GROUPS_PER_BLOCK + p * ACT_GROUPS_PER_PASS + (t >> 3);
    grp[p] = g;
    const int64_t gc = g < G ? g : G - 1;  // tail lanes re-read the last group; they store nothing
    if (!TAIL) {
      const u32x4* src = reinterpret_cast<const u32x4*>(x + gc * 128);
      raw[p][0] = __builtin_nontemporal_load(src + j);
      raw[p][1] = __builtin_nontemporal_load(src + j + 8);
    } else {
      const int64_t row = gc / Kg;
      const int c0 = (int)(gc - row * Kg) * 128 + 8 * j;   // channels c0 .. c0+7 and c0+64 ..
      const uint16_t* src = x + row * K;
      raw[p][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + min(c0, K - 8)));
      raw[p][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + min(c0 + 64, K - 8)));
      if (c0 >= K) raw[p][0] = u32x4{0u, 0u, 0u, 0u};
      if (c0 + 64 >= K) raw[p][1] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int p = 0; p < ACT_PASSES; ++p) {
    float v[16];
    unpack8(raw[p][0], v);
    unpack8(raw[p][1], v + 8);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    m = max8(m);
    const float s = group_scale(m);
    const GroupDiv d = group_div(m, s);
    if (m < 0x1p-64f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] *= d.xmul;
    }
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = quotient(v[i], d.sc, d.r);
    const u32x2 lo = u32x2{e4m3x4_q(q[0], q[1], q[2], q[3]), e4m3x4_q(q[4], q[5], q[6], q[7])};
    const u32x2 hi = u32x2{e4m3x4_q(q[8], q[9], q[10], q[11]), e4m3x4_q(q[12], q[13], q[14], q[15])};
    const int64_t g = grp[p];
    if (g < G) {
      u32x2* dst = reinterpret_cast<u32x2*>(xq + g * 128);
      __builtin_nontemporal_store(lo, dst + j);
      __builtin_nontemporal_store(hi, dst + j + 8);
      if (j == 0) xs[g] = s;
    }
  }
}

// ============================================================================
// 128x128: one workgroup per block. Thread t holds an 8x8 sub-tile: rows
// 8*(t/16) .. +7 and columns 8*(t%16) .. +7 of the block (eight 16-byte row
// loads). The block amax is reduced across the wavefront with DPP and
// shuffles, then across the four wavefronts through LDS. The optional
// transposed copy is produced by an 8x8 byte transpose in registers and an
// LDS tile.
// ============================================================================
constexpr int W_THREADS = 256;
constexpr int W_ROW_BYTES = 128 + 8;  // padded LDS row of the transposed code tile

// 4x4 byte transpose: r[i] byte j -> c[j] byte i.
__device__ __forceinline__ void transpose4x4(const uint32_t r[4], uint32_t c[4]) {
  const uint32_t p01l = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
  const uint32_t p01h = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
  const uint32_t p23l = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t p23h = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
}

// The codes are [Np, Kp] (and wq_t [Kp, Np]), N and K rounded up to 128; in
// the TAIL instantiation the rows past N and the channels past K read as +0.
// The STREAM instantiation writes the same codes in the weight-streaming
// layout instead of row-major (and no transposed copy): the block's eight
// 16-row fragments, each 2 KB in the order the MFMA's lanes hold them, meet
// in LDS and leave as eight contiguous 2 KB runs (16-byte stores).
template <bool TAIL, bool STREAM = false>
__global__ __launch_bounds__(W_THREADS) void quant_weight_128x128_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ wq, float* __restrict__ ws,
    uint8_t* __restrict__ wq_t, int N, int K, int Np, int Kp, int nb0) {
  __shared__ float red[W_THREADS / 64];
  __shared__ __align__(16) uint8_t tile_t[128 * W_ROW_BYTES];   // 17 KB: also holds the 16 KB stream tile
  const int t = threadIdx.x;
  const int kb = blockIdx.x, nb = nb0 + (int)blockIdx.y;
  const int r0 = 8 * (t >> 4), c0 = 8 * (t & 15);
  const int64_t row0 = (int64_t)nb * 128 + r0;
  const int64_t col0 = (int64_t)kb * 128 + c0;

  u32x4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!TAIL) {
      raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w + (row0 + i) * K + col0));
    } else {
      const int64_t r = min(row0 + i, (int64_t)N - 1), c = min(col0, (int64_t)K - 8);
      raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w + r * K + c));
      if (row0 + i >= N || col0 >= K) raw[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[8];
    unpack8(raw[i], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  m = max64(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = group_scale(m);
  const GroupDiv d = group_div(m, s);
  const bool tiny = m < 0x1p-64f;

  uint32_t code[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[8];
    unpack8(raw[i], v);
    if (tiny) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= d.xmul;
    }
    float q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = quotient(v[e], d.sc, d.r);
    code[i][0] = e4m3x4_q(q[0], q[1], q[2], q[3]);
    code[i][1] = e4m3x4_q(q[4], q[5], q[6], q[7]);
    if (!STREAM)
      __builtin_nontemporal_store(u32x2{code[i][0], code[i][1]},
                                  reinterpret_cast<u32x2*>(wq + (row0 + i) * Kp + col0));
  }
  if (t == 0) ws[(int64_t)nb * (Kp / 128) + kb] = s;

  if (STREAM) {
    // Row rl = r0 + i, channels c0 .. c0 + 7 of the block: fragment rl / 16,
    // lane 16 (c0 / 32) + rl % 16, half (c0 / 16) % 2, bytes c0 % 16 .. + 7.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = r0 + i;
      const int off = ((rl / 16) * 2 + (c0 / 16) % 2) * 1024 + 16 * (16 * (c0 / 32) + rl % 16) + c0 % 16;
      *reinterpret_cast<u32x2*>(tile_t + off) = u32x2{code[i][0], code[i][1]};
    }
    __syncthreads();
    const int64_t kbt = Kp / 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = t + W_THREADS * j;                 // 16-byte piece of the 16 KB tile
      const int fl = piece / 128;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tile_t + 16 * piece),
                                  reinterpret_cast<u32x4*>(wq + (((int64_t)nb * 8 + fl) * kbt + kb) * 2048 +
                                                           16 * (piece % 128)));
    }
    return;
  }

  if (wq_t != nullptr) {
    // Transpose the 8x8 byte tile: out[j] holds column c0+j, rows r0..r0+7.
    // The pieces meet in an LDS tile [column][row] and leave as 128-byte rows
    // of wq_t (eight lanes per row), so every store fills whole cache lines.
    uint32_t out[8][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {      // column bytes 0-3 / 4-7
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {          // rows 0-3 / 4-7
        uint32_t r[4], c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = code[4 * rh + i][half];
        transpose4x4(r, c);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) out[4 * half + jj][rh] = c[jj];
      }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      *reinterpret_cast<u32x2*>(tile_t + (c0 + jj) * W_ROW_BYTES + r0) = u32x2{out[jj][0], out[jj][1]};
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int row = (t >> 3) + 32 * h;   // column kb*128 + row of w
      const int seg = t & 7;
      const uint8_t* src = tile_t + row * W_ROW_BYTES + 16 * seg;
      const u32x2 a = *reinterpret_cast<const u32x2*>(src);
      const u32x2 b = *reinterpret_cast<const u32x2*>(src + 8);
      __builtin_nontemporal_store(u32x4{a[0], a[1], b[0], b[1]},
                                  reinterpret_cast<u32x4*>(wq_t + ((int64_t)kb * 128 + row) * Np +
                                                           (int64_t)nb * 128 + 16 * seg));
    }
  }
}

// ============================================================================
// 128x1 transposed: tile = 128 tokens x 128 channels per workgroup (one scale
// group along the tokens). Thread t reads channels 8*(t%16) .. +7 of tokens
// 8*(t/16) .. +7 (eight 16-byte loads; each load instruction of a wavefront
// covers four whole 256-byte token rows). Channel amax: in-thread over 8
// tokens, across the 4 lanes of a wavefront that share the channels, then
// across the 4 wavefronts through LDS. The codes go to an LDS tile
// [128 channels][128 tokens] as 8-byte pieces and leave as 128-byte rows of
// xq_t. A ragged token count M is padded: xq_t is [C, Mp] with Mp = M rounded
// up to 128, and the tokens past M are read as +0 (code 0x00). In the TAIL
// instantiation the last channel block is partial: its channels past C read
// as +0 and their rows of xq_t / xs_t are not written.
// ============================================================================
constexpr int T_THREADS = 256;
constexpr int T_CH = 128;
constexpr int T_ROW_BYTES = 128 + 8;  // padded LDS row of the transposed code tile

// Workgroup order of the 128x1 and dual kernels (grid [token blocks, channel
// blocks]): token_major_block_of in tile_map.h. Every tensor has fewer than
// 2^40 elements and a workgroup covers 2^14, so the ids fit in int.
__device__ __forceinline__ void token_major_block(int& mb, int& cbi) {
  const int nx = (int)gridDim.x, n = nx * (int)gridDim.y;
  token_major_block_of((int)blockIdx.x + (int)blockIdx.y * nx, nx, n, mb, cbi);
}

template <bool TAIL>
__global__ __launch_bounds__(T_THREADS) void transpose_quant_128x1_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq_t, float* __restrict__ xs_t,
    int M, int C, int cb0) {
  __shared__ float red[4][T_CH];
  __shared__ float p_sc[T_CH], p_r[T_CH], p_mul[T_CH];
  __shared__ __align__(16) uint8_t tile[T_CH * T_ROW_BYTES];

  const int t = threadIdx.x;
  const int cc = t & 15;          // channel chunk: channels 8cc .. 8cc+7 of the tile
  const int tr = 8 * (t >> 4);    // first token of this thread's eight
  const int wave = t >> 6, lane = t & 63;
  int mb, cbi;
  token_major_block(mb, cbi);
  const int64_t m0 = (int64_t)mb * 128;
  const int64_t c0 = ((int64_t)cb0 + cbi) * T_CH;
  const int64_t Mp = ((int64_t)M + 127) & ~(int64_t)127;   // padded token count of xq_t

  // tokens past M (a ragged last block) read as +0: they leave the amax
  // alone and quantize to code 0x00
  const int64_t cl = TAIL ? min(c0 + 8 * cc, (int64_t)C - 8) : c0 + 8 * cc;   // in-bounds chunk
  const bool cvalid = !TAIL || c0 + 8 * cc < C;
  u32x4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + tr + i;
    raw[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(x + min(row, (int64_t)M - 1) * C + cl));
    if (row >= M || !cvalid) raw[i] = u32x4{0u, 0u, 0u, 0u};
  }

  float v[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack8(raw[i], v[i]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float mm = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mm = fmaxf(mm, fabsf(v[i][e]));
    // lanes with equal (lane % 16) share channels: reduce over lane bits 4..5
    mm = fmaxf(mm, __shfl_xor(mm, 16, 64));
    mm = fmaxf(mm, __shfl_xor(mm, 32, 64));
    if (lane < 16) red[wave][8 * lane + e] = mm;
  }
  __syncthreads();
  if (t < T_CH) {
    const int c = t;
    const float m = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    const float s = group_scale(m);
    const GroupDiv d = group_div(m, s);
    p_sc[c] = d.sc;
    p_r[c] = d.r;
    p_mul[c] = d.xmul;
    if (!TAIL || c0 + c < C) xs_t[(c0 + c) * (Mp / 128) + mb] = s;
  }
  __syncthreads();

#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * cc + e;
    const float sc = p_sc[c], r = p_r[c], mul = p_mul[c];
    float xv[8], q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = v[i][e];
    if (wave_any(mul != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] *= mul;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quotient(xv[i], sc, r);
    *reinterpret_cast<u32x2*>(tile + c * T_ROW_BYTES + tr) =
        u32x2{e4m3x4_q(q[0], q[1], q[2], q[3]), e4m3x4_q(q[4], q[5], q[6], q[7])};
  }
  __syncthreads();

  // 128 rows x 128 bytes = 1024 16-byte pieces, four per thread, 8 lanes per row.
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = (t >> 3) + 32 * h;
    const int seg = t & 7;
    const uint8_t* src = tile + row * T_ROW_BYTES + 16 * seg;
    const u32x2 a = *reinterpret_cast<const u32x2*>(src);
    const u32x2 b = *reinterpret_cast<const u32x2*>(src + 8);
    if (!TAIL || c0 + row < C)
      __builtin_nontemporal_store(u32x4{a[0], a[1], b[0], b[1]},
                                  reinterpret_cast<u32x4*>(xq_t + (c0 + row) * Mp + m0 + 16 * seg));
  }
}

// ============================================================================
// Produce-and-quantize: one read of a tile of 128 tokens x 128 channels
// produces bf16 values and emits their 1x128 row groups (xq, xs; as
// quantize_act_1x128) and, optionally, their 128x1 token groups written
// transposed (xq_t, xs_t; as transpose_quantize_128x1). The producer is
//   EW_COPY     the input itself (the dual quantizer);
//   EW_RMSNORM  y = bf16(fl32(fl32(x * rstd[m]) * gamma[c]));
//   EW_SWIGLU   y = bf16(fl32(silu(g) * u)), silu(g) = g * rcp(1 + exp2(-g * log2(e)))
//               with the hardware exp2 and reciprocal (relative error ~2^-21).
// Thread layout and the transposed half are those of the 128x1 kernel; a row
// group's amax is this thread's 8 channels reduced over the 16 lanes that
// share its 8 tokens (one DPP row). M may be ragged: rows past M are read
// clamped, produce +0, and only the padded transposed copy [C, Mp] (Mp = M
// rounded up to 128) holds their 0x00 codes. In the TAIL instantiation the
// last channel block is partial: channels past C produce +0, the 1x128 codes
// are written padded ([M, Cp], Cp = C rounded up to 128, 0x00 past C), and the
// transposed rows past C are not written.
// ============================================================================
enum EwOp { EW_COPY = 0, EW_RMSNORM = 1, EW_SWIGLU = 2 };

struct EwArgs {
  const uint16_t* x;      // bf16 [M, C]: input (COPY), x (RMSNORM) or gate g (SWIGLU)
  const uint16_t* x2;     // bf16 [M, C]: up projection u (SWIGLU)
  const uint16_t* gamma;  // bf16 [C] (RMSNORM)
  const float* rstd;      // fp32 [M] (RMSNORM)
  uint16_t* y;            // bf16 [M, C] copy of the produced values, or null
  uint8_t* xq;
  float* xs;
  uint8_t* xq_t;          // null: no 128x1 output
  float* xs_t;
  int M, C, Cp, cb0;      // Cp: C rounded up to 128 (row length of xq)
};

template <int OP, bool TAIL>
__global__ __launch_bounds__(T_THREADS) void ew_quant_kernel(EwArgs a) {
  __shared__ float red[4][T_CH];
  __shared__ float p_sc[T_CH], p_r[T_CH], p_mul[T_CH];
  __shared__ __align__(16) uint8_t tile[T_CH * T_ROW_BYTES];

  const int t = threadIdx.x;
  const int cc = t & 15;          // channel chunk: channels 8cc .. 8cc+7 of the tile
  const int tr = 8 * (t >> 4);    // first token of this thread's eight
  const int wave = t >> 6, lane = t & 63;
  int mb, cbi;
  token_major_block(mb, cbi);
  const int cb = a.cb0 + cbi;
  const int64_t m0 = (int64_t)mb * 128;
  const int64_t c0 = (int64_t)cb * T_CH;
  const int C = a.C;
  const int64_t cl = TAIL ? min(c0 + 8 * cc, (int64_t)C - 8) : c0 + 8 * cc;   // in-bounds chunk
  const bool cvalid = !TAIL || c0 + 8 * cc < C;

  u32x4 raw[8], raw2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = min(m0 + tr + i, (int64_t)a.M - 1);
    raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x + row * C + cl));
    if (OP == EW_SWIGLU)
      raw2[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x2 + row * C + cl));
  }

  // The produced values are bf16 numbers; they stay packed (two per
  // register) and are widened where used, which halves the registers held
  // across the two quantizing passes.
  u32x4 pv[8];
  if (OP == EW_COPY) {
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = raw[i];
  } else if (OP == EW_RMSNORM) {
    float gm[8];
    unpack8(*reinterpret_cast<const u32x4*>(a.gamma + cl), gm);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = a.rstd[min(m0 + tr + i, (int64_t)a.M - 1)];
      float xv[8], yv[8];
      unpack8(raw[i], xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] = (xv[e] * r) * gm[e];
      pv[i] = u32x4{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                    pack_bf16x2(yv[6], yv[7])};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float gv[8], uv[8], yv[8];
      unpack8(raw[i], gv);
      unpack8(raw2[i], uv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // sigmoid with the hardware exp2 and reciprocal (each within ~1 ulp):
        // exp(-g) overflowing to inf gives g * 0 = -0 for very negative g
        const float ex = __builtin_amdgcn_exp2f(gv[e] * -1.44269504088896341f);
        const float sg = gv[e] * __builtin_amdgcn_rcpf(1.0f + ex);
        yv[e] = sg * uv[e];
      }
      pv[i] = u32x4{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                    pack_bf16x2(yv[6], yv[7])};
    }
  }
  // tokens past M (a ragged last block) and channels past C (a partial last
  // channel block) are +0: they leave every amax alone and quantize to 0x00
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (m0 + tr + i >= a.M || !cvalid) pv[i] = u32x4{0u, 0u, 0u, 0u};
  auto val = [&](int i, int e) -> float {
    const uint32_t w = pv[i][e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  };
  if (OP != EW_COPY && a.y != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = m0 + tr + i;
      if (row < a.M && cvalid) __builtin_nontemporal_store(pv[i], reinterpret_cast<u32x4*>(a.y + row * C + c0 + 8 * cc));
    }
  }

  // ---- 1x128 row groups: token m0+tr+i, channels c0 .. c0+127 ----
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(val(i, e)));
    m = max16(m);
    const float s = group_scale(m);
    const GroupDiv d = group_div(m, s);
    float xv[8], q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = val(i, e);
    if (wave_any(d.xmul != 1.0f)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] *= d.xmul;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = quotient(xv[e], d.sc, d.r);
    const int64_t row = m0 + tr + i;
    if (row < a.M) {
      __builtin_nontemporal_store(u32x2{e4m3x4_q(q[0], q[1], q[2], q[3]), e4m3x4_q(q[4], q[5], q[6], q[7])},
                                  reinterpret_cast<u32x2*>(a.xq + row * a.Cp + c0 + 8 * cc));
      if (cc == 0) a.xs[row * (a.Cp / 128) + cb] = s;
    }
  }
  if (a.xq_t == nullptr) return;   // uniform over the workgroup

  // ---- 128x1 token groups, written transposed into [C, Mp] ----
  const int64_t Mp = ((int64_t)a.M + 127) & ~(int64_t)127;   // padded token count of xq_t
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float mm = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mm = fmaxf(mm, fabsf(val(i, e)));
    mm = fmaxf(mm, __shfl_xor(mm, 16, 64));
    mm = fmaxf(mm, __shfl_xor(mm, 32, 64));
    if (lane < 16) red[wave][8 * lane + e] = mm;
  }
  __syncthreads();
  if (t < T_CH) {
    const int c = t;
    const float m = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    const float s = group_scale(m);
    const GroupDiv d = group_div(m, s);
    p_sc[c] = d.sc;
    p_r[c] = d.r;
    p_mul[c] = d.xmul;
    if (!TAIL || c0 + c < C) a.xs_t[(c0 + c) * (Mp / 128) + mb] = s;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * cc + e;
    const float sc = p_sc[c], r = p_r[c], mul = p_mul[c];
    float xv[8], q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = val(i, e);
    if (wave_any(mul != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] *= mul;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quotient(xv[i], sc, r);
    *reinterpret_cast<u32x2*>(tile + c * T_ROW_BYTES + tr) =
        u32x2{e4m3x4_q(q[0], q[1], q[2], q[3]), e4m3x4_q(q[4], q[5], q[6], q[7])};
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = (t >> 3) + 32 * h;
    const int seg = t & 7;
    const uint8_t* src = tile + row * T_ROW_BYTES + 16 * seg;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8);
    if (!TAIL || c0 + row < C)
      __builtin_nontemporal_store(u32x4{lo[0], lo[1], hi[0], hi[1]},
                                  reinterpret_cast<u32x4*>(a.xq_t + (c0 + row) * Mp + m0 + 16 * seg));
  }
}

// ============================================================================
// RMSNorm statistics: rstd[m] = 1 / sqrt(fl32(sum_k x[m,k]^2 / K) + eps), one
// wavefront per row. Each lane accumulates its 16-byte chunks in order with
// fmaf; the 64 lane sums are added in a fixed butterfly, so the result is
// deterministic.
// ============================================================================
__global__ __launch_bounds__(256) void rms_rstd_kernel(const uint16_t* __restrict__ x,
                                                       float* __restrict__ rstd, int64_t M, int K,
                                                       float eps, int64_t blk0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (blk0 + blockIdx.x) * 4 + wave;
  if (row >= M) return;   // uniform per wavefront
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * K);
  float acc = 0.0f;
  for (int c = lane; c < K / 8; c += 64) {
    float v[8];
    unpack8(__builtin_nontemporal_load(src + c), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(v[e], v[e], acc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) rstd[row] = 1.0f / sqrtf(acc / (float)K + eps);
}

// ============================================================================
// Plain encoder: 4 fp32 values -> 4 E4M3 bytes per thread.
// ============================================================================
__global__ __launch_bounds__(256) void cast_f32_e4m3_kernel(const f32x4* __restrict__ in,
                                                          uint32_t* __restrict__ out, int64_t n4,
                                                          int64_t blk0) {
  const int64_t i = (blk0 + blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) {
    const f32x4 v = in[i];
    out[i] = e4m3x4(v[0], v[1], v[2], v[3]);
  }
}

// ============================================================================
// Launchers (shapes validated by the caller).
// ============================================================================
static int64_t groups128(int64_t n) { return (n + 127) / 128; }

hipError_t launch_quant_act_1x128(const void* x, int64_t M, int64_t K, uint8_t* xq, float* xs,
                                  hipStream_t stream) {
  const int64_t Kg = groups128(K);
  const int64_t G = M * Kg;
  const int64_t blocks = (G + ACT_GROUPS_PER_BLOCK - 1) / ACT_GROUPS_PER_BLOCK;
  const bool tail = K % 128 != 0;
  for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks1D) {
    const int64_t nb = blocks - b0 < kMaxBlocks1D ? blocks - b0 : kMaxBlocks1D;
    if (tail)
      hipLaunchKernelGGL(quant_act_1x128_kernel<true>, dim3((unsigned)nb), dim3(ACT_THREADS), 0, stream,
                         static_cast<const uint16_t*>(x), xq, xs, G, b0, (int)K, (int)Kg);
    else
      hipLaunchKernelGGL(quant_act_1x128_kernel<false>, dim3((unsigned)nb), dim3(ACT_THREADS), 0, stream,
                         static_cast<const uint16_t*>(x), xq, xs, G, b0, (int)K, (int)Kg);
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight_128x128(const void* w, int64_t N, int64_t K, uint8_t* wq, float* ws,
                                       uint8_t* wq_t, hipStream_t stream) {
  const int64_t nbt = groups128(N), kbt = groups128(K);
  const bool tail = N % 128 != 0 || K % 128 != 0;
  for (int64_t y0 = 0; y0 < nbt; y0 += kMaxGridY) {
    const int64_t ny = nbt - y0 < kMaxGridY ? nbt - y0 : kMaxGridY;
    const dim3 grid((unsigned)kbt, (unsigned)ny);
    if (tail)
      hipLaunchKernelGGL(quant_weight_128x128_kernel<true>, grid, dim3(W_THREADS), 0, stream,
                         static_cast<const uint16_t*>(w), wq, ws, wq_t, (int)N, (int)K, (int)(nbt * 128),
                         (int)(kbt * 128), (int)y0);
    else
      hipLaunchKernelGGL(quant_weight_128x128_kernel<false>, grid, dim3(W_THREADS), 0, stream,
                         static_cast<const uint16_t*>(w), wq, ws, wq_t, (int)N, (int)K, (int)N, (int)K, (int)y0);
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight_stream(const void* w, int64_t N, int64_t K, uint8_t* wq_s, float* ws,
                                      hipStream_t stream) {
  const int64_t nbt = groups128(N), kbt = groups128(K);
  const bool tail = N % 128 != 0 || K % 128 != 0;
  for (int64_t y0 = 0; y0 < nbt; y0 += kMaxGridY) {
    const int64_t ny = nbt - y0 < kMaxGridY ? nbt - y0 : kMaxGridY;
    const dim3 grid((unsigned)kbt, (unsigned)ny);
    if (tail)
      hipLaunchKernelGGL((quant_weight_128x128_kernel<true, true>), grid, dim3(W_THREADS), 0, stream,
                         static_cast<const uint16_t*>(w), wq_s, ws, nullptr, (int)N, (int)K, (int)(nbt * 128),
                         (int)(kbt * 128), (int)y0);
    else
      hipLaunchKernelGGL((quant_weight_128x128_kernel<false, true>), grid, dim3(W_THREADS), 0, stream,
                         static_cast<const uint16_t*>(w), wq_s, ws, nullptr, (int)N, (int)K, (int)N, (int)K,
                         (int)y0);
  }
  return hipGetLastError();
}

// Grid: token blocks along x (adjacent workgroups write adjacent 128-byte
// pieces of the same xq_t rows), channel blocks along y.
hipError_t launch_transpose_quant_128x1(const void* x, int64_t M, int64_t C, uint8_t* xq_t,
                                        float* xs_t, hipStream_t stream) {
  const int64_t nc = groups128(C);
  for (int64_t y0 = 0; y0 < nc; y0 += kMaxGridY) {
    const int64_t ny = nc - y0 < kMaxGridY ? nc - y0 : kMaxGridY;
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)ny);
    if (C % 128)
      hipLaunchKernelGGL(transpose_quant_128x1_kernel<true>, grid, dim3(T_THREADS), 0, stream,
                         static_cast<const uint16_t*>(x), xq_t, xs_t, (int)M, (int)C, (int)y0);
    else
      hipLaunchKernelGGL(transpose_quant_128x1_kernel<false>, grid, dim3(T_THREADS), 0, stream,
                         static_cast<const uint16_t*>(x), xq_t, xs_t, (int)M, (int)C, (int)y0);
  }
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_ew(EwArgs a, int64_t M, int64_t C, hipStream_t stream) {
  const int64_t nc = groups128(C);
  for (int64_t y0 = 0; y0 < nc; y0 += kMaxGridY) {
    const int64_t ny = nc - y0 < kMaxGridY ? nc - y0 : kMaxGridY;
    a.cb0 = (int)y0;
    const dim3 grid((unsigned)((M + 127) / 128), (unsigned)ny);
    if (C % 128)
      hipLaunchKernelGGL((ew_quant_kernel<OP, true>), grid, dim3(T_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((ew_quant_kernel<OP, false>), grid, dim3(T_THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

static EwArgs ew_args(const void* x, int64_t M, int64_t C, uint8_t* xq, float* xs, uint8_t* xq_t,
                      float* xs_t) {
  EwArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.xq = xq; a.xs = xs; a.xq_t = xq_t; a.xs_t = xs_t;
  a.M = (int)M; a.C = (int)C; a.Cp = (int)(groups128(C) * 128);
  return a;
}

hipError_t launch_quant_dual(const void* x, int64_t M, int64_t C, uint8_t* xq, float* xs,
                             uint8_t* xq_t, float* xs_t, hipStream_t stream) {
  return launch_ew<EW_COPY>(ew_args(x, M, C, xq, xs, xq_t, xs_t), M, C, stream);
}

hipError_t launch_rmsnorm_quant(const void* x, const void* gamma, float eps, int64_t M, int64_t K,
                                float* rstd, void* y, uint8_t* xq, float* xs, uint8_t* xq_t,
                                float* xs_t, hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks1D) {
    const int64_t nb = blocks - b0 < kMaxBlocks1D ? blocks - b0 : kMaxBlocks1D;
    hipLaunchKernelGGL(rms_rstd_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), rstd, M, (int)K, eps, b0);
  }
  EwArgs a = ew_args(x, M, K, xq, xs, xq_t, xs_t);
  a.gamma = static_cast<const uint16_t*>(gamma);
  a.rstd = rstd;
  a.y = static_cast<uint16_t*>(y);
  return launch_ew<EW_RMSNORM>(a, M, K, stream);
}

hipError_t launch_swiglu_quant(const void* gate, const void* up, int64_t M, int64_t N, void* h,
                               uint8_t* hq, float* hs, uint8_t* hq_t, float* hs_t, hipStream_t stream) {
  EwArgs a = ew_args(gate, M, N, hq, hs, hq_t, hs_t);
  a.x2 = static_cast<const uint16_t*>(up);
  a.y = static_cast<uint16_t*>(h);
  return launch_ew<EW_SWIGLU>(a, M, N, stream);
}

hipError_t launch_cast_f32_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  const int64_t blocks = (n4 + 255) / 256;
  for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks1D) {
    const int64_t nb = blocks - b0 < kMaxBlocks1D ? blocks - b0 : kMaxBlocks1D;
    hipLaunchKernelGGL(cast_f32_e4m3_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                       reinterpret_cast<const f32x4*>(in), reinterpret_cast<uint32_t*>(out), n4, b0);
  }
  return hipGetLastError();
}

}  // namespace fp8bsq
