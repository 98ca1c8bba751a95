// ssm_conv.hip - gfx950 kernels of the causal depthwise convolution (width 4) and
// SiLU that sit in front of the selective scan in the Mamba block, for whole
// sequences and for one decode token.
//
//   out[b,d,t] = silu(bias[d] + sum_{k<4} w[d,k] * x[b,d,t-3+k])
//
// with the inputs before t = 0 taken from a conv state (the last 3 inputs of the
// previous segment, oldest first) or zeros. The block layout -- projection, a
// channel-wise Conv1d of width d_conv = 4, SiLU, then the SSM -- is in "Mamba
// Architecture Explained" (sivaro), section "The Architecture in Practice"; the
// printed layer has no padding, the causal left padding by 3 is the reading taken
// here (it keeps the output as long as the input and never looks ahead).
//
// Both kernels move a few bytes per (token, channel) and do 4 FMAs, an exp and a
// reciprocal on them: they are HBM-bound. The sequence kernel gives each thread 16
// consecutive tokens of one row (two 16-byte bf16 loads and stores, coalesced along
// the row) and reads the 3-token halo from the 8 bytes before them, which the
// neighbouring thread has just pulled into the cache.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kW = 4;        // taps
constexpr int kRun = 16;     // tokens per thread

__device__ __forceinline__ float silu_c(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * 1.4426950408889634f));
}
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const uint16_t* p) {
    return __uint_as_float((uint32_t)*p << 16);
}
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(uint16_t* p, float v) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)v);   // round to nearest even
}

// 8 values <-> registers: one 16-byte access (bf16) or two (fp32). x and y are touched
// once per launch, so these go through the streaming (non-temporal) path, which keeps
// the caches for the halo reads and saves about 8% of the kernel's time on gfx950.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
    const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
    const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2_t f = {v[2 * i], v[2 * i + 1]};
        w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    }
    const u32x4_t o = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store8(float* p, const float* v) {
    const f32x4_t a = {v[0], v[1], v[2], v[3]};
    const f32x4_t b = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(p + 4));
}
// the 3 inputs before an aligned run of 8: one 8-byte (bf16) or 16-byte (fp32) load of
// the 4 before it
__device__ __forceinline__ void load_halo(const uint16_t* p, float* v) {
    const uint2 u = *reinterpret_cast<const uint2*>(p - 4);
    v[0] = __uint_as_float(u.x & 0xffff0000u);
    v[1] = __uint_as_float(u.y << 16);
    v[2] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load_halo(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p - 4);
    v[0] = a.y; v[1] = a.z; v[2] = a.w;
}

// One thread = 16 consecutive tokens of one (batch, channel) row.
template <typename IO>
__global__ __launch_bounds__(256) void conv1d_fwd_kernel(const ConvParams p) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t runs = (p.seqlen + kRun - 1) / kRun;
    if (i >= p.rows * runs) return;
    const int64_t row = i / runs;
    const int64_t t0 = (i - row * runs) * kRun;
    const int64_t d = row % p.dim;
    const IO* xr = static_cast<const IO*>(p.x) + row * p.seqlen;
    IO* yr = static_cast<IO*>(p.y) + row * p.seqlen;
    const IO* sr = p.state_in ? static_cast<const IO*>(p.state_in) + row * (kW - 1) : nullptr;
    const int n = (p.seqlen - t0 < kRun) ? (int)(p.seqlen - t0) : kRun;
    const bool vec = p.aligned && n == kRun;

    // win[j] = x[t0 - 3 + j], j < 19
    float win[kW - 1 + kRun];
    if (t0 >= kW - 1 && p.aligned) {
        load_halo(xr + t0, win);
    } else {
#pragma unroll
        for (int j = 0; j < kW - 1; ++j) {
            const int64_t t = t0 - (kW - 1) + j;
            win[j] = t >= 0 ? ld(xr + t) : (sr ? ld(sr + (kW - 1) + t) : 0.0f);
        }
    }
    if (vec) {
#pragma unroll
        for (int q = 0; q < kRun; q += 8) load8(xr + t0 + q, win + kW - 1 + q);
    } else {
#pragma unroll
        for (int j = 0; j < kRun; ++j) win[kW - 1 + j] = j < n ? ld(xr + t0 + j) : 0.0f;
    }
    const float4 w = *reinterpret_cast<const float4*>(p.w + d * kW);
    const float bias = p.bias ? p.bias[d] : 0.0f;
    float out[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
        float a = bias;
        a = __builtin_fmaf(w.x, win[j], a);
        a = __builtin_fmaf(w.y, win[j + 1], a);
        a = __builtin_fmaf(w.z, win[j + 2], a);
        a = __builtin_fmaf(w.w, win[j + 3], a);
        out[j] = p.silu ? silu_c(a) : a;
    }
    if (vec) {
#pragma unroll
        for (int q = 0; q < kRun; q += 8) store8(yr + t0 + q, out + q);
    } else {
#pragma unroll
        for (int j = 0; j < kRun; ++j)
            if (j < n) st(yr + t0 + j, out[j]);
    }
    // the last run of the row writes the new state: the last 3 of [state, x], which
    // are win[n .. n+2] (for a row shorter than 3 they reach back into the old state)
    if (p.state_out && t0 + n == p.seqlen) {
        IO* so = static_cast<IO*>(p.state_out) + row * (kW - 1);
#pragma unroll
        for (int j = 0; j < kW - 1; ++j) {
            float v = win[j];
#pragma unroll
            for (int m = 1; m <= kRun; ++m)
                if (n == m) v = win[m + j];
            st(so + j, v);
        }
    }
}

// The decode update. A workgroup of 256 threads owns 512 consecutive (batch, channel)
// rows; thread i owns rows 2i and 2i+1. The rows' states (3 values each) are
// contiguous, so they move between HBM and LDS with full-width coalesced accesses
// (192 threads x 16 bytes in bf16) and each thread reads and writes its 6 values in
// LDS. Everything a thread needs from HBM is requested before the first barrier: the
// kernel is short, so its time is mostly the latency of one round of loads and one
// of stores, and many small workgroups keep many of them in flight.
constexpr int kRows = 2;
constexpr int kBlockRows = 256 * kRows;
constexpr int kChunks = kBlockRows * (kW - 1) / 8;   // 8-value pieces of a block's states

template <typename IO> struct Vec;
template <> struct Vec<uint16_t> {   // 8 bf16 = 16 bytes
    static __device__ __forceinline__ void copy(uint16_t* dst, const uint16_t* src) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
    static __device__ __forceinline__ void load2(const uint16_t* p, float* v) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        v[0] = __uint_as_float(u << 16);
        v[1] = __uint_as_float(u & 0xffff0000u);
    }
};
template <> struct Vec<float> {      // 8 fp32 = 32 bytes
    static __device__ __forceinline__ void copy(float* dst, const float* src) {
        *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
        *reinterpret_cast<float4*>(dst + 4) = *reinterpret_cast<const float4*>(src + 4);
    }
    static __device__ __forceinline__ void load2(const float* p, float* v) {
        const float2 a = *reinterpret_cast<const float2*>(p);
        v[0] = a.x;
        v[1] = a.y;
    }
};

template <typename IO>
__global__ __launch_bounds__(256) void conv1d_update_kernel(const ConvParams p) {
    __shared__ __attribute__((aligned(16))) IO sst[kBlockRows * (kW - 1)];
    const int tid = threadIdx.x;
    const int64_t rb = (int64_t)blockIdx.x * kBlockRows;
    const int nb = (p.rows - rb < kBlockRows) ? (int)(p.rows - rb) : kBlockRows;
    const bool full = nb == kBlockRows && p.aligned;
    IO* gs = static_cast<IO*>(p.state_out) + rb * (kW - 1);
    const int ne = nb * (kW - 1);
    const int r0 = tid * kRows;                      // first row of this thread (in block)
    const int nr = (nb - r0 < kRows) ? (nb - r0 > 0 ? nb - r0 : 0) : kRows;
    const IO* xp = static_cast<const IO*>(p.x) + rb + r0;
    IO* yp = static_cast<IO*>(p.y) + rb + r0;

    // every load up front: x, weights, bias, and the block's states into LDS
    float xv[kRows];
    if (full) {
        Vec<IO>::load2(xp, xv);
    } else {
#pragma unroll
        for (int j = 0; j < kRows; ++j) xv[j] = j < nr ? ld(xp + j) : 0.0f;
    }
    float4 w[kRows];
    float bias[kRows];
    {
        int64_t d = (rb + r0) % p.dim;
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            w[j] = *reinterpret_cast<const float4*>(p.w + d * kW);
            bias[j] = p.bias ? p.bias[d] : 0.0f;
            if (++d == p.dim) d = 0;
        }
    }
    if (full) {
        if (tid < kChunks) Vec<IO>::copy(sst + 8 * tid, gs + 8 * tid);
    } else {
        for (int e = tid; e < ne; e += 256) sst[e] = gs[e];
    }
    __syncthreads();

    float sv[kRows * (kW - 1)], out[kRows];
#pragma unroll
    for (int e = 0; e < kRows * (kW - 1); ++e)
        sv[e] = e < nr * (kW - 1) ? ld(sst + r0 * (kW - 1) + e) : 0.0f;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float a = bias[j];
        a = __builtin_fmaf(w[j].x, sv[j * 3 + 0], a);
        a = __builtin_fmaf(w[j].y, sv[j * 3 + 1], a);
        a = __builtin_fmaf(w[j].z, sv[j * 3 + 2], a);
        a = __builtin_fmaf(w[j].w, xv[j], a);
        out[j] = p.silu ? silu_c(a) : a;
        // shift: the state of row j becomes (s1, s2, x)
        sv[j * 3 + 0] = sv[j * 3 + 1];
        sv[j * 3 + 1] = sv[j * 3 + 2];
        sv[j * 3 + 2] = xv[j];
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j)
        if (j < nr) st(yp + j, out[j]);
#pragma unroll
    for (int e = 0; e < kRows * (kW - 1); ++e)
        if (e < nr * (kW - 1)) st(sst + r0 * (kW - 1) + e, sv[e]);
    __syncthreads();
    // LDS -> HBM, contiguous
    if (full) {
        if (tid < kChunks) Vec<IO>::copy(gs + 8 * tid, sst + 8 * tid);
    } else {
        for (int e = tid; e < ne; e += 256) gs[e] = sst[e];
    }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_conv1d_fwd(const ConvParams& prm, bool bf16, hipStream_t stream) {
    const int64_t threads = prm.rows * cdiv(prm.seqlen, kRun);
    const dim3 grid((unsigned)cdiv(threads, 256));
    if (bf16)
        hipLaunchKernelGGL(conv1d_fwd_kernel<uint16_t>, grid, dim3(256), 0, stream, prm);
    else
        hipLaunchKernelGGL(conv1d_fwd_kernel<float>, grid, dim3(256), 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_conv1d_update(const ConvParams& prm, bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)cdiv(prm.rows, kBlockRows));
    if (bf16)
        hipLaunchKernelGGL(conv1d_update_kernel<uint16_t>, grid, dim3(256), 0, stream, prm);
    else
        hipLaunchKernelGGL(conv1d_update_kernel<float>, grid, dim3(256), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace ssm
