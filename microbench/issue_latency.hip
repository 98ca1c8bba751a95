// Latency probe: one wave per SIMD (1024 waves of 64), dependent vs independent VALU chains.
#include <hip/hip_runtime.h>
#include <cstdio>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

template <int CH, int KIND>
__global__ __launch_bounds__(64) void chain_k(float* __restrict__ out, int iters) {
  float v[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) v[j] = 0.3f + 0.01f * j + 1e-6f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (KIND == 0) v[j] = __builtin_fmaf(v[j], 0.999f, 0.0001f);        // fma chain
        if (KIND == 1) v[j] = __builtin_amdgcn_exp2f(-v[j]);               // exp chain
        if (KIND == 2) v[j] = __builtin_amdgcn_exp2f(v[j] * -0.7f);        // mul -> exp chain
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) s += v[j];
  out[blockIdx.x * 64 + threadIdx.x] = s;
}

template <int CH, int KIND>
int run(float* out, const char* name, int ops_per_elem) {
  const int blocks = 1024, iters = 4096;
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL((chain_k<CH, KIND>), dim3(blocks), dim3(64), 0, 0, out, iters);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  hipLaunchKernelGGL((chain_k<CH, KIND>), dim3(blocks), dim3(64), 0, 0, out, iters);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  double instr_per_wave = (double)iters * 8 * CH * ops_per_elem;
  printf("%-22s chains=%d  %8.3f ms  %6.2f cycles per instruction per wave (2.4 GHz)\n", name, CH, ms,
         ms * 1e-3 * 2.4e9 / instr_per_wave);
  return 0;
}

int main() {
  float* o; CK(hipMalloc(&o, 1024 * 64 * sizeof(float)));
  run<1, 0>(o, "fma dependent", 1); run<2, 0>(o, "fma", 1); run<4, 0>(o, "fma", 1); run<8, 0>(o, "fma", 1);
  run<1, 1>(o, "exp dependent", 1); run<2, 1>(o, "exp", 1); run<4, 1>(o, "exp", 1); run<8, 1>(o, "exp", 1);
  run<1, 2>(o, "mul+exp dependent", 2); run<4, 2>(o, "mul+exp", 2); run<8, 2>(o, "mul+exp", 2);
  CK(hipFree(o));
  printf("lat done\n");
  return 0;
}
