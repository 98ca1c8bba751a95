// Issue-rate probe: FP32 VOP2 (v_fmac, VGPR operands) with 1..8 waves per SIMD, and a mix
// where half the waves run v_exp_f32 and half run v_fmac (does the transcendental of one
// wave overlap the VOP2 work of another?).
#include <hip/hip_runtime.h>
#include <cstdio>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

template <int MODE>   // 0: fmac only; 1: exp only; 2: even waves exp, odd waves fmac
__global__ __launch_bounds__(64) void k(const float* __restrict__ in, float* __restrict__ out, int iters) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  float v[8], w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { v[j] = in[(t + j * 7) & 1023]; w[j] = in[(t * 3 + j) & 1023]; }
  const bool do_exp = MODE == 1 || (MODE == 2 && (blockIdx.x & 1) == 0);
  if (do_exp) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("v_exp_f32_e32 %0, %1" : "=v"(v[j]) : "v"(v[j]));
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(v[j]) : "v"(w[j]), "v"(w[(j + 1) & 7]));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += v[j];
  out[t] = s;
}

template <int MODE>
int run(const float* in, float* out, int waves_per_simd, const char* name) {
  const int blocks = 1024 * waves_per_simd, iters = 4096;
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL((k<MODE>), dim3(blocks), dim3(64), 0, 0, in, out, iters);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  hipLaunchKernelGGL((k<MODE>), dim3(blocks), dim3(64), 0, 0, in, out, iters);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  const double instr_per_simd = (double)waves_per_simd * iters * 8;
  printf("%-22s waves/SIMD=%d  %8.3f ms  %5.2f cycles per wave-instr per SIMD\n", name, waves_per_simd, ms,
         ms * 1e-3 * 2.4e9 / instr_per_simd);
  return 0;
}

int main() {
  float *in, *o; CK(hipMalloc(&in, 1024 * 4)); CK(hipMalloc(&o, 1024 * 8 * 64 * 4));
  CK(hipMemset(in, 0, 1024 * 4));
  for (int w : {1, 2, 3, 4, 8}) run<0>(in, o, w, "v_fmac only");
  for (int w : {1, 2, 4}) run<1>(in, o, w, "v_exp only");
  for (int w : {2, 4, 8}) run<2>(in, o, w, "half exp, half fmac");
  CK(hipFree(in)); CK(hipFree(o));
  printf("dual_issue done\n");
  return 0;
}
