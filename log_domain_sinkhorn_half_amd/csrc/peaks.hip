// Peak-rate microbenchmarks for MI355X (gfx950): the denominators of the
// half-step kernels' rooflines, measured rather than assumed.
//
//  * exp:  independent chains of v_exp_f32 (x <- 2^-x stays in (0, 1)), 8 per
//          thread, at full occupancy: the transcendental issue rate.
//  * bf16: independent chains of v_mfma_f32_32x32x16_bf16 (4 accumulators per
//          wave): the dense bf16 matrix rate.
//  * fp32: the same with v_mfma_f32_32x32x2_f32: the dense fp32 matrix rate.
//
// C ABI (a measurement utility, not part of the solver library):
//   int sk_peak(int which, int blocks, int iters, float* ms, double* ops)
// runs kernel `which` (0 exp, 1 bf16 MFMA, 2 fp32 MFMA) on `blocks` workgroups
// of 256 threads for `iters` loop trips, after one warm-up launch, and returns
// the elapsed time of the timed launch (HIP events) and the operations it did
// (exps or flops).  Returns 0 on success, else the HIP error code.  Allocates
// one small result buffer per call (each thread writes one value, so the work
// cannot be removed by the compiler).
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void k_peak_exp(float seed, int iters, float* __restrict__ out) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = seed + 0.01f * (float)(threadIdx.x + k);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_peak_bf16(float seed, int iters, float* __restrict__ out) {
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(seed * (float)(k + 1));
    b[k] = (__bf16)(seed * (float)(8 - k));
  }
  f16v c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int o = 0; o < 16; ++o) c[j][o] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int o = 0; o < 16; ++o) s += c[j][o];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_peak_fp32(float seed, int iters, float* __restrict__ out) {
  const float a = seed, b = seed * 0.5f;
  f16v c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int o = 0; o < 16; ++o) c[j][o] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int o = 0; o < 16; ++o) s += c[j][o];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

extern "C" int sk_peak(int which, int blocks, int iters, float* ms, double* ops) {
  if (which < 0 || which > 2 || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24) || !ms || !ops)
    return (int)hipErrorInvalidValue;
  float* out = nullptr;
  hipError_t e = hipMalloc(&out, sizeof(float) * 256 * (size_t)blocks);
  if (e != hipSuccess) return (int)e;
  hipEvent_t t0, t1;
  hipEventCreate(&t0);
  hipEventCreate(&t1);
  auto launch = [&](int n) {
    if (which == 0) hipLaunchKernelGGL(k_peak_exp, dim3(blocks), dim3(256), 0, 0, 0.5f, n, out);
    if (which == 1) hipLaunchKernelGGL(k_peak_bf16, dim3(blocks), dim3(256), 0, 0, 0.001f, n, out);
    if (which == 2) hipLaunchKernelGGL(k_peak_fp32, dim3(blocks), dim3(256), 0, 0, 0.001f, n, out);
  };
  launch(iters);  // warm-up
  hipEventRecord(t0, 0);
  launch(iters);
  hipEventRecord(t1, 0);
  e = hipEventSynchronize(t1);
  if (e == hipSuccess) e = hipGetLastError();
  float t = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, t0, t1);
  *ms = t;
  const double threads = 256.0 * blocks, waves = threads / 64.0;
  if (which == 0) *ops = threads * iters * 8.0;                         // exps
  if (which == 1) *ops = waves * iters * 4.0 * (2.0 * 32 * 32 * 16);   // flops
  if (which == 2) *ops = waves * iters * 4.0 * (2.0 * 32 * 32 * 2);
  hipEventDestroy(t0);
  hipEventDestroy(t1);
  hipFree(out);
  return (int)e;
}
