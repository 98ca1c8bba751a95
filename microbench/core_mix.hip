// The scan's core instruction mix per (token, state): d = Delta*a; e = exp2(d);
// b = B*u; h = e*h + b; p = C*h  -> 1 v_exp_f32 + 4 VGPR-operand VOP2 ops, with S states
// per lane (S independent recurrences), run with W waves per SIMD. Reports SIMD cycles per
// (token, state) per wave, i.e. the per-SIMD cost of one lane-row of recurrence work.
#include <hip/hip_runtime.h>
#include <cstdio>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

template <int S>
__global__ __launch_bounds__(64) void k(const float* __restrict__ in, float* __restrict__ out, int tokens) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  float a[S], h[S], p = 0.f;
#pragma unroll
  for (int j = 0; j < S; ++j) { a[j] = -0.1f * (j + 1) - 1e-6f * (t & 63); h[j] = 0.f; }
  float D = in[t & 1023] * 1e-3f + 0.01f, U = in[(t + 1) & 1023], B = in[(t + 2) & 1023], C = in[(t + 3) & 1023];
  for (int it = 0; it < tokens; ++it) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const float e = __builtin_amdgcn_exp2f(D * a[j]);
      h[j] = __builtin_fmaf(e, h[j], B * U);
      p = __builtin_fmaf(C, h[j], p);
    }
    D += 1e-7f; U = U * 0.999f; B = B + 1e-6f; C = C * 1.0001f;   // per-token operands change
  }
  float s = p;
#pragma unroll
  for (int j = 0; j < S; ++j) s += h[j];
  out[t] = s;
}

template <int S>
int run(const float* in, float* out, int w) {
  const int blocks = 1024 * w, tokens = 2048;
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL((k<S>), dim3(blocks), dim3(64), 0, 0, in, out, tokens);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  hipLaunchKernelGGL((k<S>), dim3(blocks), dim3(64), 0, 0, in, out, tokens);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  const double ts_per_simd = (double)w * tokens * S;   // wave-(token,state) units per SIMD
  printf("states/lane=%d waves/SIMD=%d  %8.3f ms  %6.2f SIMD cycles per wave-(token,state)\n", S, w, ms,
         ms * 1e-3 * 2.4e9 / ts_per_simd);
  return 0;
}

int main() {
  float *in, *o; CK(hipMalloc(&in, 1024 * 4)); CK(hipMalloc(&o, 1024 * 8 * 64 * 4));
  CK(hipMemset(in, 0, 1024 * 4));
  for (int w : {1, 2, 3, 4, 5, 6}) run<1>(in, o, w);
  for (int w : {1, 2, 3, 4}) run<2>(in, o, w);
  for (int w : {1, 2}) run<4>(in, o, w);
  CK(hipFree(in)); CK(hipFree(o));
  printf("core_mix done\n");
  return 0;
}
