// ssm_device.h - element-wise device helpers shared by the library's HIP sources
// (softplus, SiLU and their derivatives on the hardware exp2/log2/rcp, bf16 <-> fp32,
// streaming accesses, a wait for outstanding memory accesses).
// Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- element-wise
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// 2^y with round-to-nearest arithmetic only, for the decays of the fp32-io kernels:
// y = n + f with n = rint(y) and |f| <= 1/2; 2^f from its Taylor series (f ln 2)^k / k!
// up to k = 7 (truncation below 6e-9 relative on |f| <= 1/2), Horner with fused
// multiply-adds; then the exact scaling by 2^n. Error within ~1.2 ulp and without a
// systematic sign (mean relative error ~1e-10 over y in [-10, 0]). The hardware
// v_exp_f32 is as close per call but not unbiased, and a state with a long memory
// multiplies hundreds of decays: on the Mamba-2.8B layer shape in fp32 its bias alone
// takes the worst row's final state to ~1.5e-5 relative, this exp keeps it near 4e-6.
__device__ __forceinline__ float exp2_unbiased(float y) {
    y = (y < -160.0f) ? -160.0f : ((y > 128.0f) ? 128.0f : y);
    const float n = __builtin_rintf(y);
    const float f = y - n;   // exact
    float p = 1.5252733804059841e-05f;
    p = __builtin_fmaf(p, f, 1.5403530393381609e-04f);
    p = __builtin_fmaf(p, f, 1.3333558146428443e-03f);
    p = __builtin_fmaf(p, f, 9.6181291076284772e-03f);
    p = __builtin_fmaf(p, f, 5.5504108664821580e-02f);
    p = __builtin_fmaf(p, f, 2.4022650695910071e-01f);
    p = __builtin_fmaf(p, f, 6.9314718055994531e-01f);
    p = __builtin_fmaf(p, f, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

// The decay exp(Delta A) = 2^y of a kernel with io type IO: the unbiased form for fp32
// io (whose results are held to 1e-5), the hardware exp for bf16 io.
template <typename IO> __device__ __forceinline__ float decay_exp2(float y) {
    if constexpr (sizeof(IO) == 4) return exp2_unbiased(y);
    else return fast_exp2(y);
}

// softplus(v) = max(v, 0) + log1p(e^-|v|). log1p(e) is taken as log(w) + (e - (w - 1))
// with w = 1 + e rounded: the second term restores what the rounding of 1 + e lost
// (w - 1 is exact for w in [1, 2]), so small e keeps full relative accuracy.
__device__ __forceinline__ float softplus_f(float v) {
    const float e = fast_exp2(-__builtin_fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    const float r = e - (w - 1.0f);
    const float lp = __builtin_fmaf(fast_log2(w), kLn2, r);
    return __builtin_fmaxf(v, 0.0f) + lp;
}

// silu(z) = z / (1 + e^-z); for z -> -inf the exp overflows to inf, rcp gives 0.
__device__ __forceinline__ float silu_f(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // RNE
}
// Streaming (non-temporal) 16-byte load and store, for data touched exactly once per
// launch: they keep the caches for data that is reused.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream4(float* p, float a, float b, float c, float d) {
    const f32x4_t v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

// Raw buffer accesses: a 128-bit resource held in scalar registers (base address, byte
// extent, and the format word of a raw buffer on this GPU family), a 32-bit per-lane byte
// offset and a uniform one, so that an access needs no 64-bit address arithmetic per lane.
// An access past the extent reads zero and writes nothing.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ void store_one(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_one(uint16_t* p, float v) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Wait until every vector-memory access the wave has issued is complete (vmcnt 0; the
// export and LDS/scalar counters untouched: their fields at the maximum). gfx950 counts
// loads and stores with one counter, so once stores are in flight behind prefetched
// loads, the wait the compiler puts before a use of those loads waits for the stores
// too -- and it also keeps such a wait at the top of a loop whose entry has loads in
// flight. The tile loops take this wait themselves, where only accesses issued long
// before are outstanding.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// sigma(v) = 1 / (1 + e^-v): the derivative of softplus
__device__ __forceinline__ float sigmoid_f(float v) {
    return fast_rcp(1.0f + fast_exp2(-v * kLog2e));
}

// d silu / dz = s (1 + z (1 - s)) with s = sigma(z)
__device__ __forceinline__ float dsilu_f(float z) {
    const float s = sigmoid_f(z);
    return s * __builtin_fmaf(z, 1.0f - s, 1.0f);
}

// Index of the packed sequence that holds token t: the largest s in [0, nseq) with
// cu[s] <= t (0 when there is none). Reads only cu[0..nseq-1], whatever cu holds.
__device__ __forceinline__ int seq_of(const int32_t* cu, int nseq, int64_t t) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

}  // namespace dev
}  // namespace ssm
