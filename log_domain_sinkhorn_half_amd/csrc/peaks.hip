// Peak-rate microbenchmarks for MI355X (gfx950): the denominators of the
// half-step kernels' rooflines, measured rather than assumed.
//
//  * exp:  independent chains of v_exp_f32 (x <- 2^-x stays in (0, 1)), 8 per
//          thread, at full occupancy: the transcendental issue rate.
//  * bf16: independent chains of v_mfma_f32_32x32x16_bf16 (4 accumulators per
//          wave): the dense bf16 matrix rate.
//  * fp32: the same with v_mfma_f32_32x32x2_f32: the dense fp32 matrix rate.
//  * exp+add:     each exp also feeds one fp32 add into a running sum (the
//                 fp32 half-step's VALU work per score).
//  * fma+exp+add: each exp's argument comes from an fp32 FMA and its result
//                 feeds an add (the bf16 half-step's work per score).
//    Their rates (exps/s) against the exp rate show how far the adds and FMAs
//    issue beside the transcendental unit.
//  * tile: the bf16 half-step's work per key tile at d = 128 with no memory
//          traffic: two accumulators (32 queries each) x 8 chained
//          v_mfma_f32_32x32x16_bf16 (K = 128) from a per-tile start value, then
//          the 32 scores per lane through (fma, exp, add), a workgroup barrier
//          every 4 tiles; at 2 waves per SIMD (512 workgroups) as the kernel
//          runs.  Its flop rate is the most the half-step's tile structure can
//          reach when the matrix and vector streams overlap as far as the
//          hardware lets them.
//
// C ABI (a measurement utility, not part of the solver library):
//   int sk_peak(int which, int blocks, int iters, float* ms, double* ops)
// runs kernel `which` (0 exp, 1 bf16 MFMA, 2 fp32 MFMA, 3 exp+add, 4 fma+exp+add, 5 tile) on `blocks` workgroups
// of 256 threads for `iters` loop trips, after one warm-up launch, and returns
// the elapsed time of the timed launch (HIP events) and the operations it did
// (exps or flops).  Returns 0 on success, else the HIP error code.  Allocates
// one small result buffer per call (each thread writes one value, so the work
// cannot be removed by the compiler).
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

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

__global__ __launch_bounds__(256) void k_peak_exp_add(float seed, int iters, float* __restrict__ out) {
  float x[8], s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[k] = seed + 0.01f * (float)(threadIdx.x + k);
    s[k] = 0.f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = __builtin_amdgcn_exp2f(-x[k]);
      s[k] += x[k];
    }
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) t += x[k] + s[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = t;
}

// a and b come from the host, so the FMA cannot fold into a source modifier
__global__ __launch_bounds__(256) void k_peak_fma_exp_add(float seed, float a, float b, int iters,
                                                          float* __restrict__ out) {
  float x[8], s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[k] = seed + 0.01f * (float)(threadIdx.x + k);
    s[k] = 0.f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = __builtin_amdgcn_exp2f(fmaf(x[k], a, b));
      s[k] += x[k];
    }
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) t += x[k] + s[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = t;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_peak_tile(float seed, float lam2,
                                                                                          float m, int iters,
                                                                                          float* __restrict__ out) {
  // bf16 operands near 1 (distinct per lane, query tile and K step)
  u4v bq[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = 0x3c003c00u + (uint32_t)((threadIdx.x + 7 * c + 3 * i) & 0x3f);
      bq[c][i] = u4v{h, h ^ 0x10u, h ^ 0x20u, h ^ 0x30u};
    }
  float s[2] = {0.f, 0.f};
  float start = seed;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f16v acc[2];
      start += 1e-7f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int o = 0; o < 16; ++o) acc[c][o] = start + 0.001f * (float)o;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bq[0][i]),
                                                           __builtin_bit_cast(bf16x8, bq[c][i]), acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float e[16];
#pragma unroll
        for (int o = 0; o < 16; ++o) e[o] = __builtin_amdgcn_exp2f(fmaf(acc[c][o], lam2, -m));
#pragma unroll
        for (int w = 1; w < 16; w *= 2)
#pragma unroll
          for (int o = 0; o + w < 16; o += 2 * w) e[o] += e[o + w];
        s[c] += e[0];
      }
    }
    __syncthreads();
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1];
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
  if (which < 0 || which > 5 || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24) || !ms || !ops)
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
    if (which == 3) hipLaunchKernelGGL(k_peak_exp_add, dim3(blocks), dim3(256), 0, 0, 0.5f, n, out);
    if (which == 4) hipLaunchKernelGGL(k_peak_fma_exp_add, dim3(blocks), dim3(256), 0, 0, 0.5f, -0.999f, -0.001f, n, out);
    if (which == 5) hipLaunchKernelGGL(k_peak_tile, dim3(blocks), dim3(256), 0, 0, 0.25f, 0.01f, 1.f, n, out);
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
  if (which == 0 || which == 3 || which == 4) *ops = threads * iters * 8.0;  // exps
  if (which == 5) *ops = waves * (double)((iters + 3) / 4 * 4) * 16.0 * (2.0 * 32 * 32 * 16);  // flops
  if (which == 1) *ops = waves * iters * 4.0 * (2.0 * 32 * 32 * 16);   // flops
  if (which == 2) *ops = waves * iters * 4.0 * (2.0 * 32 * 32 * 2);
  hipEventDestroy(t0);
  hipEventDestroy(t1);
  hipFree(out);
  return (int)e;
}
