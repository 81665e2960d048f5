// Sustained matrix-core rate on this device at its running clock, for the
// measurement side of the roofline: independent accumulator chains per wave,
// operands in registers, no memory traffic inside the loop, so the only limit
// is how fast the matrix cores retire the instruction.
//
//   kind 0: v_mfma_i32_32x32x32_i8                 (65536 INT8 ops each)
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4, FP4  (131072 FP4 flops each)
//
// Each thread writes one word derived from its accumulators so the chains are
// live; the words themselves mean nothing.
#include "tabit_internal.h"

namespace tabit {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;    // independent accumulators per wave
constexpr int kThreads = 256;
constexpr int kWgPerCu = 4;   // four waves per SIMD: the fastest of 1, 2, 4 on MI355X

__global__ void __launch_bounds__(kThreads)
mfma_i8_probe_kernel(int iters, int seed, int* __restrict__ sink) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const v4i a = {t ^ seed, t + seed, t * 3, seed};
  const v4i b = {seed, t, t ^ 7, t + 1};
  v16i acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16i{};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
  int s = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s ^= acc[c][0] ^ acc[c][15];
  sink[t] = s;
}

__global__ void __launch_bounds__(kThreads)
mfma_fp4_probe_kernel(int iters, int seed, int* __restrict__ sink) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const v8i a = {t ^ seed, t + seed, t * 3, seed, 0, 0, 0, 0};
  const v8i b = {seed, t, t ^ 7, t + 1, 0, 0, 0, 0};
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0, 127);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][15];
  sink[t] = __float_as_int(s);
}

}  // namespace

size_t mfma_probe_sink_ints(int num_cus) { return (size_t)num_cus * kWgPerCu * kThreads; }

// kWgPerCu workgroups of four waves per CU, `iters` rounds of kChains MFMAs
// per wave.  Returns the matrix-core operations the launch performs.
double launch_mfma_probe(int kind, int iters, int num_cus, int* sink, hipStream_t s,
                         hipEvent_t ev0, hipEvent_t ev1, hipError_t* err) {
  const dim3 grid(num_cus * kWgPerCu), block(kThreads);
  const double waves = (double)num_cus * kWgPerCu * (kThreads / 64);
  if (kind == 0)
    hipExtLaunchKernelGGL(mfma_i8_probe_kernel, grid, block, 0, s, ev0, ev1, 0, iters, 1, sink);
  else
    hipExtLaunchKernelGGL(mfma_fp4_probe_kernel, grid, block, 0, s, ev0, ev1, 0, iters, 1, sink);
  *err = hipGetLastError();
  return waves * iters * kChains * (kind == 0 ? 65536.0 : 131072.0);
}

}  // namespace tabit
