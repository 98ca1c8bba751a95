// Probe: device copy / read bandwidth at 64 MiB - 2 GiB working sets, and FP32 FMA vs v_exp_f32 throughput.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

__global__ void copy_k(const float4* __restrict__ a, float4* __restrict__ b, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) b[i] = a[i];
}
__global__ void read_k(const float4* __restrict__ a, float* __restrict__ out, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  float s = 0.f;
  for (; i < n; i += stride) { float4 v = a[i]; s += v.x + v.y + v.z + v.w; }
  out[blockIdx.x * (size_t)blockDim.x + threadIdx.x] = s;
}
// MODE 0: 8 fma chains; 1: 8 exp chains; 2: 8 exp chains + 32 fma (4 per exp); 3: 8 exp + 16 fma
template <int MODE>
__global__ void alu_k(float* __restrict__ out, int iters) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  float e[8], f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { e[j] = 0.1f + 0.01f * j + 1e-7f * tid; f[j] = 0.5f + 0.01f * j; }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (MODE == 0) { f[j] = __builtin_fmaf(f[j], 0.999f, 0.001f); }
      if (MODE >= 1) { e[j] = __builtin_amdgcn_exp2f(-e[j]); }
      if (MODE == 2) {
        f[j] = __builtin_fmaf(f[j], 0.999f, 0.001f); f[j] = __builtin_fmaf(f[j], 0.999f, 0.002f);
        f[j] = __builtin_fmaf(f[j], 0.999f, 0.003f); f[j] = __builtin_fmaf(f[j], 0.999f, 0.004f);
      }
      if (MODE == 3) {
        f[j] = __builtin_fmaf(f[j], 0.999f, 0.001f); f[j] = __builtin_fmaf(f[j], 0.999f, 0.002f);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += e[j] + f[j];
  out[tid] = s;
}

template <int MODE>
int run_alu(float* out, int blocks, int iters, double ops_per_iter_thread, const char* name) {
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL(alu_k<MODE>, dim3(blocks), dim3(256), 0, 0, out, iters);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(alu_k<MODE>, dim3(blocks), dim3(256), 0, 0, out, iters);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b)); ms /= 5;
  double lanes = (double)blocks * 256;
  printf("%-28s %8.3f ms  %8.2f T lane-iter-ops/s  (per thread-iter ops=%g)\n", name, ms,
         lanes * iters * ops_per_iter_thread / (ms * 1e-3) / 1e12, ops_per_iter_thread);
  return 0;
}

int main() {
  int dev; CK(hipGetDevice(&dev));
  hipDeviceProp_t pr; CK(hipGetDeviceProperties(&pr, dev));
  printf("device %s  CUs %d  clock %d kHz  l2 %d  gcnArch %s\n", pr.name, pr.multiProcessorCount, pr.clockRate, pr.l2CacheSize, pr.gcnArchName);
  // copy / read bandwidth at 2 GiB and 64 MiB working sets
  const size_t big = (size_t)2 << 30;
  float4 *a, *b; float* o;
  CK(hipMalloc(&a, big)); CK(hipMalloc(&b, big)); CK(hipMalloc(&o, 64 << 20));
  CK(hipMemset(a, 0, big)); CK(hipMemset(b, 0, big));
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  for (size_t bytes : {(size_t)64 << 20, (size_t)128 << 20, (size_t)1 << 30, big}) {
    size_t n = bytes / 16;
    int blocks = 256 * 16;
    hipLaunchKernelGGL(copy_k, dim3(blocks), dim3(256), 0, 0, a, b, n); CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(e0, 0));
    for (int r = 0; r < 10; ++r) hipLaunchKernelGGL(copy_k, dim3(blocks), dim3(256), 0, 0, a, b, n);
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    float ms; CK(hipEventElapsedTime(&ms, e0, e1)); ms /= 10;
    printf("copy %6zu MiB: %8.3f ms  %8.1f GB/s (read+write)\n", bytes >> 20, ms, 2.0 * bytes / (ms * 1e-3) / 1e9);
    hipLaunchKernelGGL(read_k, dim3(blocks), dim3(256), 0, 0, a, o, n); CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(e0, 0));
    for (int r = 0; r < 10; ++r) hipLaunchKernelGGL(read_k, dim3(blocks), dim3(256), 0, 0, a, o, n);
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1)); ms /= 10;
    printf("read %6zu MiB: %8.3f ms  %8.1f GB/s\n", bytes >> 20, ms, 1.0 * bytes / (ms * 1e-3) / 1e9);
  }
  // ALU: 256 CUs x 32 blocks of 256 threads (8 waves per SIMD); o holds 64 MiB >= threads*4 B
  const int blocks = 256 * 32;
  const int iters = 2048;
  if ((size_t)blocks * 256 * 4 > ((size_t)64 << 20)) { printf("out too small\n"); return 1; }
  run_alu<0>(o, blocks, iters, 8, "fma x8");
  run_alu<1>(o, blocks, iters, 8, "exp x8");
  run_alu<2>(o, blocks, iters, 40, "exp x8 + fma x32");
  run_alu<3>(o, blocks, iters, 24, "exp x8 + fma x16");
  CK(hipFree(a)); CK(hipFree(b)); CK(hipFree(o));
  printf("probe done\n");
  return 0;
}
