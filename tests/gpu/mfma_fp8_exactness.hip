// How exactly does one gfx950 FP8 MFMA sum its 128 products?
//
// The GEMM kernels compute each 128-long K block of a 16 x 16 output tile with
// one v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3, zero accumulator), through
// the same builtin and operand layout as below, and then scale and promote
// that partial sum in fp32. The products of two E4M3 values are exact in
// fp32, but the matrix core need not add them exactly. This program measures
// how far one such MFMA lands from the exact sum, on fixed operand sets:
//
//   narrow  values {0, +-112, +-224, +-448}: every partial sum is a small
//           multiple of 112^2, so an exact adder and fp32 agree bit for bit;
//   wide    values k/4 (k/4 <= 16, at most 4 significant bits, random sign)
//           with one +-448 per row at a row-dependent position, so some
//           outputs hold a 448 x 448 product among small ones (the value set
//           of the wide exact-operand GEMM tests);
//   two     exactly two nonzero products per output: +-448 x 448 plus
//           2^e x 2^f, e, f in -9..6, sweeping the small product from 2^-18
//           to 2^12;
//   cancel  64 products +-448 x 448 that cancel exactly, plus 64 small
//           products (powers of two 2^-9 .. 2^-2, random sign);
//   reach   448 x 448 at K position 0 and 1 x 0.25 at position p (row i of
//           A holds its 1 at p = REACH_POS[i]; columns j of B with odd j have
//           no 448): whether a small product at position p is cut against a
//           large one at position 0, i.e. which positions the matrix core
//           aligns together.
//
// Exact sums are formed on the host in double: a product of two E4M3 values
// has at most 8 significant bits and lies in [2^-18, 448^2], so any sum of
// 128 of them is exact in double's 53 bits whatever the order.
//
// Output, one line per class:
//   class=<name> outputs=<n> equal_rne=<n> max_dev_over_maxprod=<r> log2=<l>
//       worst: i j gpu=<hex> exact=<value> maxprod=<value>
// and, for the "two" and "reach" classes, one line per output:
//   two i j small=<2^(e+f)> gpu=<hex> exact=<value> rne=<hex>
//   reach i j pos=<p> gpu=<hex> exact=<value> rne=<hex>
// Exit status 0 when it ran (the test reads the printed values).
//
// Build (done by the package build): hipcc --offload-arch=gfx950 -O3 <this> -o <binary>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#define CHECK(call)                                                               \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      return 2;                                                                   \
    }                                                                             \
  } while (0)

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16 * 128;   // bytes of one 16-row, 128-long operand

// One 64-lane wavefront per case. Lane (r = lane % 16, g = lane / 16) holds
// bytes 32g .. 32g+31 of row r of each operand (the GEMM kernels' fragment
// layout); result element t of the lane is D[4g + t][r] (row of A, row of B).
__global__ __launch_bounds__(64) void one_mfma(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                               float* __restrict__ D) {
  const int c = blockIdx.x, lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const u32x4* pa = reinterpret_cast<const u32x4*>(A + (size_t)c * kTile + r * 128 + 32 * g);
  const u32x4* pb = reinterpret_cast<const u32x4*>(B + (size_t)c * kTile + r * 128 + 32 * g);
  const u32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
  for (int t = 0; t < 4; ++t) D[(size_t)c * 256 + (4 * g + t) * 16 + r] = d[t];
}

// OCP E4M3 value of a byte (finite codes only are used here).
static double e4m3_value(uint8_t b) {
  const int E = (b >> 3) & 15, T = b & 7;
  const double mag = E == 0 ? T * ldexp(1.0, -9) : (8 + T) * ldexp(1.0, E - 10);
  return (b & 0x80) ? -mag : mag;
}

// The byte of an exactly representable value (search of the finite codes).
static uint8_t e4m3_code(double v) {
  for (int b = 0; b < 256; ++b) {
    if ((b & 0x7F) == 0x7F) continue;
    if (e4m3_value((uint8_t)b) == v && !(v == 0.0 && b != 0)) return (uint8_t)b;
  }
  printf("no E4M3 code for %g\n", v);
  return 0;
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {   // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

struct Class {
  const char* name;
  int first, count;   // cases
};

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main() {
  std::vector<Class> classes;
  std::vector<uint8_t> A, B;
  auto new_case = [&]() {
    A.resize(A.size() + kTile, 0);
    B.resize(B.size() + kTile, 0);
    return (int)(A.size() / kTile) - 1;
  };
  auto at = [&](std::vector<uint8_t>& M, int c, int row, int k) -> uint8_t& { return M[(size_t)c * kTile + row * 128 + k]; };

  // narrow
  {
    const double vals[4] = {0.0, 112.0, 224.0, 448.0};
    const int first = (int)(A.size() / kTile);
    for (int n = 0; n < 16; ++n) {
      const int c = new_case();
      for (int row = 0; row < 16; ++row)
        for (int k = 0; k < 128; ++k) {
          const double va = vals[rnd() % 4] * ((rnd() & 1) ? -1 : 1);
          const double vb = vals[rnd() % 4] * ((rnd() & 1) ? -1 : 1);
          at(A, c, row, k) = e4m3_code(va);
          at(B, c, row, k) = e4m3_code(vb);
        }
    }
    classes.push_back({"narrow", first, 16});
  }
  // wide: k/4 up to 16 with at most 4 significant bits, one +-448 per row
  {
    std::vector<double> grid;
    for (int k = 0; k <= 64; ++k) {
      int odd = k;
      while (odd && odd % 2 == 0) odd /= 2;
      if (odd < 16) grid.push_back(k / 4.0);
    }
    const int first = (int)(A.size() / kTile);
    for (int n = 0; n < 64; ++n) {
      const int c = new_case();
      for (int row = 0; row < 16; ++row) {
        const int ka = (7 * row + n) % 128, kb = (7 * row + n + (row & 1)) % 128;
        for (int k = 0; k < 128; ++k) {
          double va = k == ka ? 448.0 : grid[rnd() % grid.size()];
          double vb = k == kb ? 448.0 : grid[rnd() % grid.size()];
          if (rnd() & 1) va = -va;
          if (rnd() & 1) vb = -vb;
          at(A, c, row, k) = e4m3_code(va);
          at(B, c, row, k) = e4m3_code(vb);
        }
      }
    }
    classes.push_back({"wide", first, 64});
  }
  // two: +-448 * 448 + 2^e * 2^f
  {
    const int c = new_case();
    for (int row = 0; row < 16; ++row) {
      at(A, c, row, 0) = e4m3_code(448.0);
      at(A, c, row, 1) = e4m3_code(ldexp(1.0, row - 9));
      at(B, c, row, 0) = e4m3_code((row & 1) ? -448.0 : 448.0);
      at(B, c, row, 1) = e4m3_code(ldexp(1.0, row - 9));
    }
    classes.push_back({"two", c, 1});
  }
  // cancel: 64 large products that cancel exactly, plus 64 small ones
  {
    const int first = (int)(A.size() / kTile);
    for (int n = 0; n < 8; ++n) {
      const int c = new_case();
      for (int row = 0; row < 16; ++row)
        for (int k = 0; k < 128; ++k) {
          if (k < 64) {
            at(A, c, row, k) = e4m3_code(448.0);
            at(B, c, row, k) = e4m3_code((k & 1) ? -448.0 : 448.0);
          } else {
            at(A, c, row, k) = e4m3_code(ldexp((rnd() & 1) ? -1.0 : 1.0, -9 + (int)(rnd() % 8)));
            at(B, c, row, k) = e4m3_code(ldexp((rnd() & 1) ? -1.0 : 1.0, -9 + (int)(rnd() % 8)));
          }
        }
    }
    classes.push_back({"cancel", first, 8});
  }
  // reach: 448 x 448 at position 0, 1 x 0.25 at position REACH_POS[i]
  const int REACH_POS[16] = {1, 2, 3, 4, 7, 8, 15, 16, 31, 32, 33, 63, 64, 65, 96, 127};
  {
    const int c = new_case();
    for (int row = 0; row < 16; ++row) {
      at(A, c, row, 0) = e4m3_code(448.0);
      at(A, c, row, REACH_POS[row]) = e4m3_code(1.0);
      at(B, c, row, 0) = e4m3_code((row & 1) ? 0.0 : 448.0);
      for (int k = 1; k < 128; ++k) at(B, c, row, k) = e4m3_code(0.25);
    }
    classes.push_back({"reach", c, 1});
  }

  const int ncases = (int)(A.size() / kTile);
  uint8_t *dA = nullptr, *dB = nullptr;
  float* dD = nullptr;
  CHECK(hipMalloc(&dA, A.size()));
  CHECK(hipMalloc(&dB, B.size()));
  CHECK(hipMalloc(&dD, (size_t)ncases * 256 * sizeof(float)));
  CHECK(hipMemcpy(dA, A.data(), A.size(), hipMemcpyHostToDevice));
  CHECK(hipMemcpy(dB, B.data(), B.size(), hipMemcpyHostToDevice));
  printf("cases=%d\n", ncases);
  fflush(stdout);
  hipLaunchKernelGGL(one_mfma, dim3(ncases), dim3(64), 0, 0, dA, dB, dD);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  std::vector<float> D((size_t)ncases * 256);
  CHECK(hipMemcpy(D.data(), dD, D.size() * sizeof(float), hipMemcpyDeviceToHost));

  for (const Class& cl : classes) {
    int outputs = 0, equal = 0;
    double worst = 0.0;
    int wc = -1, wi = 0, wj = 0;
    for (int c = cl.first; c < cl.first + cl.count; ++c)
      for (int i = 0; i < 16; ++i)
        for (int j = 0; j < 16; ++j) {
          double exact = 0.0, maxprod = 0.0;
          for (int k = 0; k < 128; ++k) {
            const double p = e4m3_value(at(A, c, i, k)) * e4m3_value(at(B, c, j, k));
            exact += p;
            maxprod = fmax(maxprod, fabs(p));
          }
          const float gpu = D[(size_t)c * 256 + i * 16 + j];
          const float rne = (float)exact;
          ++outputs;
          if (f32_bits(gpu) == f32_bits(rne)) ++equal;
          const double dev = maxprod > 0 ? fabs((double)gpu - exact) / maxprod : fabs((double)gpu - exact);
          if (wc < 0 || dev > worst) {
            worst = dev;
            wc = c;
            wi = i;
            wj = j;
          }
          if (!strcmp(cl.name, "two"))
            printf("two %d %d small=%.9g gpu=%08x exact=%.17g rne=%08x\n", i, j, ldexp(1.0, i + j - 18), f32_bits(gpu),
                   exact, f32_bits(rne));
          if (!strcmp(cl.name, "reach"))
            printf("reach %d %d pos=%d gpu=%08x exact=%.17g rne=%08x\n", i, j, REACH_POS[i], f32_bits(gpu), exact,
                   f32_bits(rne));
        }
    double wexact = 0.0, wmax = 0.0;
    for (int k = 0; k < 128; ++k) {
      const double p = e4m3_value(at(A, wc, wi, k)) * e4m3_value(at(B, wc, wj, k));
      wexact += p;
      wmax = fmax(wmax, fabs(p));
    }
    printf("class=%s outputs=%d equal_rne=%d max_dev_over_maxprod=%.6g log2=%.3f\n", cl.name, outputs, equal, worst,
           worst > 0 ? log2(worst) : -1000.0);
    printf("    worst: case %d i %d j %d gpu=%08x (%.17g) exact=%.17g maxprod=%.17g\n", wc, wi, wj,
           f32_bits(D[(size_t)wc * 256 + wi * 16 + wj]), (double)D[(size_t)wc * 256 + wi * 16 + wj], wexact, wmax);
  }
  CHECK(hipFree(dA));
  CHECK(hipFree(dB));
  CHECK(hipFree(dD));
  return 0;
}
