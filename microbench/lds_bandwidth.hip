// LDS bandwidth probe: 8 waves per CU-block, loops of ds_read_b128 (distinct / broadcast) and ds_read_b32.
#include <hip/hip_runtime.h>
#include <cstdio>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

template <int MODE>
__global__ __launch_bounds__(512) void lds_k(float* __restrict__ out, int iters) {
  __shared__ float buf[512 * 4 + 64];
  const int t = threadIdx.x;
  for (int i = t; i < 512 * 4 + 64; i += 512) buf[i] = (float)i;
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float a1 = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (MODE == 0) {  // distinct 16B per lane, contiguous across lanes
        const float4 v = *reinterpret_cast<const float4*>(&buf[((t + r * 64) & 511) * 4]);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      if (MODE == 1) {  // broadcast: same 16B for all lanes of the wave
        const float4 v = *reinterpret_cast<const float4*>(&buf[((r * 4 + (it & 7)) & 511) * 4]);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      if (MODE == 2) {  // distinct dword per lane
        a1 += buf[(t + r * 64 + it) & 2047];
      }
      if (MODE == 3) {  // 16 distinct dwords, rows replicated (the B/C block pattern)
        a1 += buf[((t & 15) + r * 16 + (it & 7) * 128) & 2047];
      }
    }
  }
  out[blockIdx.x * 512 + t] = acc.x + acc.y + acc.z + acc.w + a1;
}

template <int MODE>
int run(float* out, const char* name, double bytes_per_lane_op) {
  const int blocks = 512, iters = 2048;   // 2 blocks of 8 waves per CU
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL((lds_k<MODE>), dim3(blocks), dim3(512), 0, 0, out, iters);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  hipLaunchKernelGGL((lds_k<MODE>), dim3(blocks), dim3(512), 0, 0, out, iters);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  double lane_ops = (double)blocks * 512 * iters * 8;
  printf("%-34s %8.3f ms  %7.1f bytes/clk/CU delivered to lanes  (%.2f ns per wave-instr per CU)\n", name, ms,
         lane_ops * bytes_per_lane_op / (ms * 1e-3) / 256 / 2.4e9,
         ms * 1e6 / (lane_ops / 64 / 256));
  return 0;
}

int main() {
  float* o; CK(hipMalloc(&o, 512 * 512 * sizeof(float)));
  run<0>(o, "ds_read_b128 distinct", 16);
  run<1>(o, "ds_read_b128 broadcast", 16);
  run<2>(o, "ds_read_b32 distinct", 4);
  run<3>(o, "ds_read_b32 16-distinct rows repl.", 4);
  CK(hipFree(o));
  printf("lds done\n");
  return 0;
}
