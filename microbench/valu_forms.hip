#include <hip/hip_runtime.h>
#include <cstdio>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
template <int K> __device__ __forceinline__ float qp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), K, 0xF, 0xF, true));
}
template <int MODE>
__global__ __launch_bounds__(256) void form_k(const float* __restrict__ in, float* __restrict__ out, int iters, float sc) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  float v[8], w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { v[j] = in[(t + j * 7) & 1023]; w[j] = in[(t * 3 + j) & 1023]; }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (MODE == 0) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(v[j]) : "v"(w[j]), "v"(w[(j + 1) & 7]));
      if (MODE == 1) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(v[j]) : "s"(sc), "v"(w[j]));
      if (MODE == 2) asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(v[j]) : "s"(sc), "v"(v[j]));
      if (MODE == 3) asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(v[j]) : "v"(v[j]), "v"(w[j]), "v"(w[(j + 1) & 7]));
      if (MODE == 4) asm volatile("v_mul_f32_dpp %0, %1, %2 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf" : "=v"(v[j]) : "v"(w[j]), "v"(v[j]));
      if (MODE == 5) asm volatile("v_fmamk_f32 %0, %1, 0x3f7fbe77, %2" : "=v"(v[j]) : "v"(v[j]), "v"(w[j]));
      if (MODE == 6) asm volatile("v_mov_b32_dpp %0, %1 row_newbcast:5 row_mask:0xf bank_mask:0xf" : "=v"(v[j]) : "v"(w[j]));
      if (MODE == 7) asm volatile("v_exp_f32_e32 %0, %1" : "=v"(v[j]) : "v"(v[j]));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += v[j];
  out[t] = s;
}
template <int MODE>
int run(const float* in, float* out, const char* name) {
  const int blocks = 256 * 32, iters = 2048;
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL((form_k<MODE>), dim3(blocks), dim3(256), 0, 0, in, out, iters, 0.999f);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  hipLaunchKernelGGL((form_k<MODE>), dim3(blocks), dim3(256), 0, 0, in, out, iters, 0.999f);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  double wave_instr = (double)blocks * 4 * iters * 8;
  printf("%-34s %8.3f ms  %5.2f cycles per wave-instr per SIMD\n", name, ms, ms * 1e-3 * 2.4e9 * 1024 / wave_instr);
  return 0;
}
int main() {
  float *in, *o; CK(hipMalloc(&in, 1024 * 4)); CK(hipMalloc(&o, 256 * 32 * 256 * 4));
  CK(hipMemset(in, 0, 1024 * 4));
  run<0>(in, o, "v_fmac_f32_e32 v,v,v");
  run<1>(in, o, "v_fmac_f32_e32 v,s,v");
  run<2>(in, o, "v_mul_f32_e32 v,s,v");
  run<3>(in, o, "v_fma_f32 v,v,v,v (VOP3)");
  run<4>(in, o, "v_mul_f32_dpp quad_perm");
  run<5>(in, o, "v_fmamk_f32 v,v,K,v");
  run<6>(in, o, "v_mov_b32_dpp row_newbcast");
  run<7>(in, o, "v_exp_f32 (asm)");
  CK(hipFree(in)); CK(hipFree(o));
  printf("forms2 done\n");
  return 0;
}
