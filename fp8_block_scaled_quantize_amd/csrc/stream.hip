// The weight-streaming layout and the forward GEMM for decode-sized token
// counts that reads it.
//
// Source: Resumen Técnico: Jet-RL (gist.science), "Arquitectura Central" and
// "Esquema de Cuantización": rollout runs the same FP8 forward as training,
// on the 128x128-block weight codes, and the weights change only once per
// optimizer update. The layout below is a second arrangement of exactly those
// codes (made once per update, beside wq); it changes no arithmetic.
//
// Why: with at most 64 token rows the forward is bound by streaming the weight
// from HBM once. In the row-major wq [Np, Kp] a 16-row MFMA fragment of one
// 128-long K block is 16 separate 128-byte segments, Kp bytes apart, and the
// tile kernels fetch each K step as 64 such segments per workgroup. In the
// stream layout the fragment is 2 KB of contiguous bytes, already in the order
// the MFMA's lanes hold them, and the fragments of one 16-row band follow each
// other along K, so a wavefront reads its whole band as one sequential stream
// of 1 KB loads (one per load instruction) straight into its MFMA registers.
//
// Layout (Kb = Kp / 128): for 16-row fragment f, K block kb, half h in {0, 1},
// lane l = 16 g + r (g, r < 16 is the MFMA lane: row r, bytes 32g .. 32g+31 of
// the K block) and byte b < 16,
//     wq_s[((f Kb + kb) 2 + h) 1024 + 16 l + b] = wq[(16 f + r) Kp + 128 kb + 32 g + 16 h + b].
//
// The GEMM computes exactly the forward of the tile kernels: per K block one
// 16x16x128 MFMA (weight fragment as the first operand, token fragment as the
// second, zero accumulator), promoted by acc = fma(d, xs * ws, acc) in K
// order, then rounded to bf16 -- so its outputs are bit-identical to
// fp8_gemm_fwd's for every token row.
#include "device_common.h"
#include "launch.h"

namespace fp8bsq {

typedef int i32x8s __attribute__((ext_vector_type(8)));

constexpr int64_t kStreamMaxBlocks = (int64_t)1 << 22;   // workgroups of one 1-D launch at most

// ---------------------------------------------------------------------------
// wq [Np, Kp] -> wq_s: one 16-byte piece per lane; piece p of wq_s is
// (f, kb, h, l) = (p / (128 Kb), (p / 128) % Kb, (p / 64) % 2, p % 64).
// The writes are contiguous; a wavefront reads 16 rows x 4 pieces of one K
// block (its partner wavefront, the other half, the pieces in between).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void weight_stream_layout_kernel(const u32x4* __restrict__ wq,
                                                                   u32x4* __restrict__ wq_s, int64_t Kp,
                                                                   int64_t npieces, int64_t p0) {
  const int64_t p = p0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= npieces) return;
  const int64_t Kb = Kp / 128;
  const int l = (int)(p % 64), h = (int)((p / 64) % 2);
  const int64_t kb = (p / 128) % Kb, f = p / (128 * Kb);
  const int64_t row = 16 * f + (l % 16);
  const int64_t col = 128 * kb + 32 * (l / 16) + 16 * h;
  wq_s[p] = wq[(row * Kp + col) / 16];
}

hipError_t launch_weight_stream_layout(const uint8_t* wq, int64_t Np, int64_t Kp, uint8_t* wq_s,
                                       hipStream_t stream) {
  const int64_t npieces = Np * Kp / 16;
  const int64_t blocks = (npieces + 255) / 256;
  for (int64_t b0 = 0; b0 < blocks; b0 += kStreamMaxBlocks) {
    const int64_t nb = blocks - b0 < kStreamMaxBlocks ? blocks - b0 : kStreamMaxBlocks;
    hipLaunchKernelGGL(weight_stream_layout_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(wq), reinterpret_cast<u32x4*>(wq_s), Kp, npieces, b0 * 256);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward for J <= 64 token rows on the stream layout. A workgroup has W
// compute wavefronts, which own W consecutive 16-row weight fragments (W
// chosen so that the grid is whole rounds of the 256 compute units: 7 for a
// 28672-row weight), and TS staging wavefronts. The token rows (NB 16-row
// blocks, NB = ceil(J / 16)) pass through LDS a chunk of CH K blocks at a
// time, in a ring of L + 1 buffers with L chunks in flight; their 16-byte
// pieces are XOR-swizzled by row so the fragment reads are free of bank
// conflicts. Every compute unit reads the same token rows from L2 at about
// the same time, so a chunk takes a long round trip; narrow weights (little
// compute per chunk) need several chunks in flight to hide it.
//
// Each compute wavefront keeps the next ST_D K blocks of its fragment in
// flight in registers (2 KB each). Loads complete in issue order for the
// wait counter, so a wavefront that also loaded token chunks would have to
// drain its weight loads whenever a chunk had to land; the staging wavefronts
// carry those loads instead, and the compute wavefronts' main loop has no
// other loads and no branches, so their waits keep the ring outstanding.
//
// Chunk protocol (every wavefront passes the same nch barriers): chunk c
// goes to buffer c mod (L + 1). Chunk 0 is in place at barrier 0; between
// barriers c and c + 1 the compute wavefronts read chunk c while chunks up
// to c + L are on their way, chunk c + L sent after barrier c into the
// buffer whose chunk c - 1 every compute wavefront finished reading before
// barrier c (chunk L, whose buffer has held nothing, goes out before barrier
// 0); the staging wavefront that sent chunk c + 1 waits for it before
// barrier c + 1.
// ---------------------------------------------------------------------------
constexpr int ST_J = 64;     // token rows of one call at most
constexpr bool ST_NT = true; // weight loads marked non-temporal (read once)

__device__ __forceinline__ int st_swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}

struct StreamParams {
  const uint8_t* xq;   // [J, Kp]
  const float* xs;     // [J, Kb]
  const uint8_t* wq_s; // stream layout of [Np, Kp]
  const float* ws;     // [Np / 128, Kb]
  uint16_t* y;         // [J, N]
  int J, N, Np, Kp, Kb;
};

template <int W, int NB, int CH, int ST_D, int TS, int LS>
__global__ __launch_bounds__(64 * (W + TS)) void fp8_gemm_fwd_stream_kernel(StreamParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RJ = 16 * NB;                           // token rows staged
  constexpr int L = TS * LS;                            // chunks ahead of the one being read
  constexpr int NBUF = L + 1;
  static_assert(NB >= 1 && RJ <= ST_J && ST_D % CH == 0 && LS >= 1, "stream tile");
  static_assert((RJ * CH) % 64 == 0, "the staging wavefront copies a chunk's scales 64 at a time");
  __shared__ __align__(16) uint8_t qt[NBUF][CH][RJ * 128];
  __shared__ __align__(16) float qsc[NBUF][RJ * CH];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kb = p.Kb, J = p.J;
  const int nch = (Kb + CH - 1) / CH;

  if (wave >= W) {
    // ---- staging wavefront s of TS: LDS DMA, no data held in registers. A chunk is
    // CH * RJ / 8 copies of 1 KB (8 rows of one K block each, the row's
    // 16-byte pieces sent to their swizzled slots) and RJ * CH / 64 copies of
    // 4-byte scales (element e = row * CH + u). Rows past J repeat row J - 1
    // and K blocks past Kb repeat block Kb - 1 (never read for a result).
    // Offsets are 32-bit: J Kp < 2^30 bytes. Chunk c is sent by staging
    // wavefront c mod TS; each has at most LS chunks in flight (of any L
    // consecutive chunks, LS are its own), which its wait counter holds.
    constexpr int OPS = CH * RJ / 8 + RJ * CH / 64;
    static_assert(LS * OPS < 64, "copies of a staging wavefront in flight");
    static_assert(64 % CH == 0, "a lane's scale column is the same in every scale copy");
    const int s = wave - W;
    // lane parts of the offsets, the same for every chunk: token copy n
    // covers rows (8 n) mod RJ + lane / 8 of K block 8 n / RJ; scale copy n
    // covers element 64 n + lane, row (64 n + lane) / CH, column lane mod CH
    uint32_t roff[RJ / 8], soff[RJ * CH / 64];
#pragma unroll
    for (int m = 0; m < RJ / 8; ++m) {
      const int row = 8 * m + lane / 8;
      const int piece = (lane % 8) ^ ((row & 7) ^ ((row >> 3) & 1));
      roff[m] = (uint32_t)min(row, J - 1) * (uint32_t)p.Kp + (uint32_t)piece * 16u;
    }
#pragma unroll
    for (int n = 0; n < RJ * CH / 64; ++n) soff[n] = (uint32_t)min((64 * n + lane) / CH, J - 1) * (uint32_t)Kb;
    auto dma_chunk = [&](int c) {
      const int buf = c % NBUF;
      const uint32_t tbase = lds_addr(&qt[buf][0][0]);
#pragma unroll
      for (int n = 0; n < CH * RJ / 8; ++n) {
        const uint32_t kcol = (uint32_t)min(c * CH + n * 8 / RJ, Kb - 1) * 128u;   // wavefront-uniform
        dma16(p.xq, roff[n % (RJ / 8)] + kcol, tbase + 1024u * n);
      }
      const uint32_t sbase = lds_addr(&qsc[buf][0]);
      const uint32_t scol = (uint32_t)min(c * CH + lane % CH, Kb - 1);
#pragma unroll
      for (int n = 0; n < RJ * CH / 64; ++n) dma4(p.xs, 4u * (soff[n] + scol), sbase + 256u * n);
    };
    for (int c = s; c < L; c += TS) dma_chunk(c);
    if (s == 0) {
      wait_dma_keep<(LS - 1) * OPS>();                  // chunk 0 in place
      dma_chunk(L);                                     // buffer L holds no chunk yet
    }
    __syncthreads();                                    // barrier 0
    for (int c = 0; c + 1 < nch; ++c) {
      if (c > 0 && c % TS == s) dma_chunk(c + L);      // its buffer held chunk c - 1
      if ((c + 1) % TS == s) wait_dma_keep<(LS - 1) * OPS>();   // chunk c + 1 in place
      __syncthreads();                                  // barrier c + 1: chunk c + 1 in place, chunk c read
    }
    wait_dma_keep<0>();                                 // no copy into LDS outlives the workgroup
    return;
  }

  // ---- compute wavefronts
  const int nfrag = p.Np / 16;
  const int fidx = (int)blockIdx.x * W + wave;
  const bool live = fidx < nfrag;                       // wavefronts past the last fragment compute a copy, store nothing
  const int f = min(fidx, nfrag - 1);

  // weight fragment of K block kb: two 1 KB loads (halves 0 and 1) from a
  // wavefront-uniform base plus a 32-bit lane offset
  const uint8_t* wf = p.wq_s + (int64_t)f * Kb * 2048;
  const uint32_t loff = 16u * (uint32_t)lane;
  auto pload = [&](int kb) -> i32x8s {
    const uint8_t* q = wf + (int64_t)min(kb, Kb - 1) * 2048;
    const u32x4* a = reinterpret_cast<const u32x4*>(q + loff);
    const u32x4 lo = ST_NT ? __builtin_nontemporal_load(a) : a[0];
    const u32x4 hi = ST_NT ? __builtin_nontemporal_load(a + 64) : a[64];
    return i32x8s{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // block scales of this fragment's 128-row block (wavefront-uniform)
  const float* wsb = p.ws + (int64_t)(f / 8) * Kb;
  auto load_frag = [&](const uint8_t* t, int row) -> i32x8s {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(t + st_swz(row, 2 * g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(t + st_swz(row, 2 * g + 1));
    return i32x8s{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = zero;
  // one K block: the NB token fragments and scales from LDS, NB MFMAs back
  // to back, then the promotions
  auto step = [&](const i32x8s& pf, float psw, int buf, int kl) {
    i32x8s qf[NB];
    float qs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      qf[b] = load_frag(&qt[buf][kl][0], b * 16 + r16);
      qs[b] = qsc[buf][(b * 16 + r16) * CH + kl];
    }
    f32x4 d[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) d[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf, qf[b], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float cs = qs[b] * psw;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[b][r] = __builtin_fmaf(d[b][r], cs, acc[b][r]);
        // keeps the promotion in its K block: otherwise the compiler sinks the
        // promotions of a whole ring group to its end, holding every MFMA
        // result of the group in registers
        asm volatile("" : "+v"(acc[b][r]));
      }
    }
  };

  i32x8s ring[ST_D];
  float sring[ST_D];
#pragma unroll
  for (int u = 0; u < ST_D; ++u) {
    ring[u] = pload(u);
    sring[u] = wsb[min(u, Kb - 1)];
  }
  __syncthreads();                                      // barrier 0

  // Main loop: whole groups of ST_D K blocks (the ring index is a
  // compile-time constant); a slot's next fragment goes out once its MFMAs
  // have read it, into the same registers.
  int kb0 = 0;
  for (; kb0 + ST_D <= Kb; kb0 += ST_D) {
#pragma unroll
    for (int u = 0; u < ST_D; ++u) {
      const int kb = kb0 + u;
      const int c = kb / CH;
      step(ring[u], sring[u], c % NBUF, u % CH);
      ring[u] = pload(kb + ST_D);
      sring[u] = wsb[min(kb + ST_D, Kb - 1)];
      if (u % CH == CH - 1 && c + 1 < nch) __syncthreads();   // barrier c + 1
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Tail: the last Kb % ST_D K blocks, already in the ring.
#pragma unroll
  for (int u = 0; u < ST_D - 1; ++u) {
    const int kb = kb0 + u;
    if (kb < Kb) {
      const int c = kb / CH;
      step(ring[u], sring[u], c % NBUF, u % CH);
      if (u % CH == CH - 1 && c + 1 < nch) __syncthreads();   // barrier c + 1
    }
  }

  // lane holds y[j = 16 b + r16][16 f + 4 g .. + 3]
  if (live) {
    const int i = 16 * f + 4 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = b * 16 + r16;
      if (j < J && i < p.N)
        __builtin_nontemporal_store(u32x2{pack_bf16x2(acc[b][0], acc[b][1]), pack_bf16x2(acc[b][2], acc[b][3])},
                                    reinterpret_cast<u32x2*>(p.y + (int64_t)j * p.N + i));
    }
  }
#endif
}

// Wavefronts per workgroup for nfrag 16-row fragments: the fewest fragments
// on the busiest compute unit (workgroups dealt one per compute unit per
// round), then the largest W (fewer workgroups stage the tokens fewer times).
static int stream_waves(int nfrag) {
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int w = 1; w <= 7; ++w) {
    const int64_t wgs = (nfrag + w - 1) / w;
    const int64_t cost = (wgs + 255) / 256 * w;
    if (cost <= best_cost) {
      best_cost = cost;
      best = w;
    }
  }
  return best;
}

// Staging of one call, by workgroup width W and token blocks NB: K blocks
// per chunk (ch), weight ring depth per compute wavefront (d), staging
// wavefronts (ts) and chunks in flight per staging wavefront (ls). Wide
// weights keep one chunk in flight; narrow ones, whose compute wavefronts
// have less work per chunk, keep several (their LDS ring 58-135 KB), and
// with one token block a deeper weight ring (each measured the faster where
// it is used).
struct StreamCfg {
  int ch, d, ts, ls;
};
constexpr StreamCfg stream_cfg(int w, int nb) {
  if (w >= 5) return {4, 12, 1, 1};
  return nb == 1 ? StreamCfg{4, 12, 1, 6} : nb == 2 ? StreamCfg{4, 8, 2, 3} : nb == 3 ? StreamCfg{4, 8, 2, 2} : StreamCfg{4, 8, 3, 1};
}

template <int W, int NB>
static hipError_t run_stream_nb(const StreamParams& p, hipStream_t stream) {
  const int nfrag = p.Np / 16;
  constexpr StreamCfg k = stream_cfg(W, NB);
  hipLaunchKernelGGL((fp8_gemm_fwd_stream_kernel<W, NB, k.ch, k.d, k.ts, k.ls>), dim3((unsigned)((nfrag + W - 1) / W)),
                     dim3(64 * (W + k.ts)), 0, stream, p);
  return hipGetLastError();
}

template <int W>
static hipError_t run_stream(const StreamParams& p, hipStream_t stream) {
  switch ((p.J + 15) / 16) {
    case 1: return run_stream_nb<W, 1>(p, stream);
    case 2: return run_stream_nb<W, 2>(p, stream);
    case 3: return run_stream_nb<W, 3>(p, stream);
    default: return run_stream_nb<W, 4>(p, stream);
  }
}

hipError_t launch_gemm_fwd_stream(const uint8_t* xq, const float* xs, const uint8_t* wq_s, const float* ws, void* y,
                                  int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  StreamParams p{};
  p.xq = xq; p.xs = xs; p.wq_s = wq_s; p.ws = ws; p.y = static_cast<uint16_t*>(y);
  p.J = (int)M; p.N = (int)N;
  p.Np = (int)((N + 127) / 128 * 128);
  p.Kp = (int)((K + 127) / 128 * 128);
  p.Kb = p.Kp / 128;
  switch (stream_waves(p.Np / 16)) {
    case 1: return run_stream<1>(p, stream);
    case 2: return run_stream<2>(p, stream);
    case 3: return run_stream<3>(p, stream);
    case 4: return run_stream<4>(p, stream);
    case 5: return run_stream<5>(p, stream);
    case 6: return run_stream<6>(p, stream);
    default: return run_stream<7>(p, stream);
  }
}

}  // namespace fp8bsq
