// Memory-only replica of the scan's access pattern: 256 workgroups, each owning 80 rows
// of 2048 bf16 tokens (x, delta, z read; y written), streamed in chunks of CH tokens per
// row per step. No compute. Bytes moved = 4 tensors x rows x 2048 x 2.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
constexpr int ROWS = 20480, L = 2048, CGW = 80;

template <int CH>   // tokens per row per step; each thread moves 8 bytes (4 tokens)
__global__ __launch_bounds__(640) void pat_k(const uint2* __restrict__ x, const uint2* __restrict__ d,
                                             const uint2* __restrict__ z, uint2* __restrict__ y) {
  constexpr int TPR = CH / 4;                  // threads per row per step
  constexpr int RPS = 640 / TPR;               // rows covered per pass of the workgroup
  const int t = threadIdx.x;
  const int r0 = blockIdx.x * CGW;
  for (int step = 0; step < L / CH; ++step) {
    for (int rr = t / TPR; rr < CGW; rr += RPS) {
      const int64_t idx = ((int64_t)(r0 + rr) * L + step * CH + (t % TPR) * 4) / 4;
      uint2 a = x[idx], b = d[idx], c = z[idx];
      y[idx] = make_uint2(a.x ^ b.x ^ c.x, a.y ^ b.y ^ c.y);
    }
  }
}
template <int CH>
int run(const uint2* x, const uint2* d, const uint2* z, uint2* y) {
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  hipLaunchKernelGGL((pat_k<CH>), dim3(ROWS / CGW), dim3(640), 0, 0, x, d, z, y);
  CK(hipGetLastError()); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a, 0));
  for (int r = 0; r < 5; ++r) hipLaunchKernelGGL((pat_k<CH>), dim3(ROWS / CGW), dim3(640), 0, 0, x, d, z, y);
  CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b)); ms /= 5;
  double bytes = 4.0 * ROWS * L * 2;
  printf("chunk %4d tokens (%5d B/row/step): %8.1f us  %7.1f GB/s\n", CH, CH * 2, ms * 1e3, bytes / (ms * 1e-3) / 1e9);
  return 0;
}
int main() {
  const size_t n = (size_t)ROWS * L * 2;  // bytes per tensor
  uint2 *x, *d, *z, *y;
  CK(hipMalloc(&x, n)); CK(hipMalloc(&d, n)); CK(hipMalloc(&z, n)); CK(hipMalloc(&y, n));
  CK(hipMemset(x, 1, n)); CK(hipMemset(d, 2, n)); CK(hipMemset(z, 3, n));
  run<32>(x, d, z, y); run<64>(x, d, z, y); run<128>(x, d, z, y); run<256>(x, d, z, y); run<512>(x, d, z, y); run<2048>(x, d, z, y);
  CK(hipFree(x)); CK(hipFree(d)); CK(hipFree(z)); CK(hipFree(y));
  printf("pattern done\n");
  return 0;
}
