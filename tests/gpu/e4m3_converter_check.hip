// Exhaustive GPU check of the hardware E4M3 converter over the quotient range.
//
// The quantizer kernels hand their quotients q (always |q| < 449; the CPU
// proof in tests/cpu/quotient_exhaustive.c records the largest) straight to
// v_cvt_pk_fp8_f32 without first clamping them to +-448. That is sound only
// if, for every fp32 value v with |v| < 449, the converter gives the same byte
// for v as for med3(v, -448, 448). This program checks exactly that, for every
// such bit pattern and both signs (2 x 1138786304 values), and prints the
// number of mismatches (and the first few). Exit status 0 when it ran; the
// test reads the printed count.
//
// Build (done by the package build): hipcc --offload-arch=gfx950 -O3 <this> -o <binary>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#define CHECK(call)                                                               \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      return 2;                                                                   \
    }                                                                             \
  } while (0)

constexpr uint32_t kLimit = 0x43E08000u;   // bit pattern of 449.0f: all |v| < 449 lie below it
constexpr int kPerThread = 16;
constexpr int kRecord = 8;

__global__ void check(unsigned long long* counts, uint32_t* first) {
  const uint64_t base = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * kPerThread;
  unsigned long long bad = 0;
  for (int k = 0; k < kPerThread; ++k) {
    const uint64_t u = base + k;
    if (u >= kLimit) break;
    for (int neg = 0; neg < 2; ++neg) {
      const float v = __uint_as_float((uint32_t)u | (neg ? 0x80000000u : 0u));
      const int plain = __builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFF;
      const float c = __builtin_amdgcn_fmed3f(v, 448.0f, -448.0f);
      const int clamped = __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFF;
      if (plain != clamped) {
        ++bad;
        const unsigned long long slot = atomicAdd(counts + 1, 1ull);
        if (slot < kRecord) {
          first[3 * slot] = __float_as_uint(v);
          first[3 * slot + 1] = (uint32_t)plain;
          first[3 * slot + 2] = (uint32_t)clamped;
        }
      }
    }
  }
  if (bad) atomicAdd(counts, bad);
}

int main() {
  unsigned long long* counts = nullptr;
  uint32_t* first = nullptr;
  CHECK(hipMalloc(&counts, 2 * sizeof(unsigned long long)));
  CHECK(hipMalloc(&first, 3 * kRecord * sizeof(uint32_t)));
  CHECK(hipMemset(counts, 0, 2 * sizeof(unsigned long long)));
  CHECK(hipMemset(first, 0, 3 * kRecord * sizeof(uint32_t)));
  const int threads = 256;
  const uint64_t per_block = (uint64_t)threads * kPerThread;
  const uint32_t blocks = (uint32_t)((kLimit + per_block - 1) / per_block);
  printf("checking %llu values (|v| < 449, both signs)\n", 2ull * kLimit);
  fflush(stdout);
  hipLaunchKernelGGL(check, dim3(blocks), dim3(threads), 0, 0, counts, first);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  unsigned long long h[2];
  uint32_t f[3 * kRecord];
  CHECK(hipMemcpy(h, counts, sizeof(h), hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(f, first, sizeof(f), hipMemcpyDeviceToHost));
  for (unsigned i = 0; i < kRecord && i < h[1]; ++i) {
    float v;
    __builtin_memcpy(&v, &f[3 * i], 4);
    printf("  v=%08x (%.9g): unclamped byte %02x, clamped byte %02x\n", f[3 * i], v, f[3 * i + 1], f[3 * i + 2]);
  }
  printf("converter_mismatches=%llu\n", h[0]);
  CHECK(hipFree(counts));
  CHECK(hipFree(first));
  return 0;
}
