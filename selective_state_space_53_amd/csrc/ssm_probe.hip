// ssm_probe.hip - hardware probes behind the benchmark's roofline figures (libssmprobe.so,
// not part of the scan library's ABI):
//  * ssmprobe_copy / ssmprobe_read: device copy and read-only bandwidth over a caller's
//    buffers (16-byte accesses, grid-stride), the achievable-HBM reference next to the
//    8 TB/s peak; the copy also calibrates the FETCH_SIZE / WRITE_SIZE counters.
//  * ssmprobe_valu: issue cost of single VALU instructions and of the scan's core mix on
//    one SIMD, as SIMD cycles per wave64 instruction. Every wave runs a fixed count of
//    one instruction form (inline assembly: the count and the operand kinds are exact)
//    and records its start and end shader-clock counter, the real-time counter and the
//    SIMD it ran on; the host groups waves by SIMD. No memory access inside the timed loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void copy_kernel(const float4* __restrict__ src,
                                                   float4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const float4* __restrict__ src,
                                                   float* __restrict__ out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float s = 0.0f;
    for (int64_t i = t; i < n; i += stride) {
        const float4 v = src[i];
        s += (v.x + v.y) + (v.z + v.w);
    }
    out[t] = s;   // keeps the loads; out has gridDim.x * blockDim.x floats
}

// 16 independent register chains; every asm statement is exactly one instruction.
#define P16(M) M(0) M(1) M(2) M(3) M(4) M(5) M(6) M(7) M(8) M(9) M(10) M(11) M(12) M(13) M(14) M(15)

enum Kind {
    kFmacVV = 0,    // v_fmac_f32 acc, vb, vc           (VOP2, VGPR operands)
    kMulVV = 1,     // v_mul_f32 acc, acc, vb           (VOP2)
    kFmaVop3 = 2,   // v_fma_f32 acc, acc, vb, vc       (VOP3)
    kFmacSV = 3,    // v_fmac_f32 acc, sb, vc           (VOP2, one SGPR operand)
    kExp = 4,       // v_exp_f32 acc, vb                (transcendental, independent)
    kAddDpp = 5,    // v_add_f32_dpp acc, acc, acc row_shr:1
    kCoreMix = 6,   // the scan's core, 2 states per lane: per token 2 x (v_mul, v_exp),
                    // 2 x (v_mul, v_fmac) for the update, v_mul + v_fmac for the readout
    kExpFmac4 = 7,  // 1 v_exp_f32 then 4 independent v_fmac_f32 (VGPR), repeated
    kCoreStruct = 8,// the core with structured decays (no exp): per token 2 x v_mul for
                    // the decays, 2 x (v_mul, v_fmac) update, v_mul + v_fmac readout
    kPermSwap16 = 9,// v_permlane16_swap_b32 a, b (gfx950: odd 16-lane rows of a <-> even
                    // rows of b), on 8 independent register pairs
    kCndmask = 10,  // v_cndmask_b32 acc, acc, vb, vcc
    kCndmaskS = 11, // v_cndmask_b32_e64 acc, acc, vb, s[pair]   (VOP3, SGPR-pair condition)
    kBfi = 12,      // v_bfi_b32 acc, vmask, vb, acc             (VOP3, VGPR operands)
    kCmpCnd = 13,   // v_cmp_lt_i32 vcc, vlane, vk then v_cndmask_b32 acc, 0, acc, vcc:
                    // the compare-and-select pair the compiler emits for a per-lane test
    kNumKinds = 14
};

// instructions per loop iteration, by kind
__host__ __device__ constexpr int instr_per_iter(int kind) {
    return kind == kCoreMix ? 80 : kind == kExpFmac4 ? 80 : kind == kCoreStruct ? 64 : 64;
}

template <int KIND>
__global__ __launch_bounds__(256) void valu_kernel(int iters, uint64_t* __restrict__ rec,
                                                   float* __restrict__ sink, float seed,
                                                   int sb) {
    const int lane = threadIdx.x & 63;
    float a0, a1, a2, a3, a4, a5, a6, a7, a8, a9, a10, a11, a12, a13, a14, a15;
#define INIT(i) a##i = seed + (float)(lane + i) * 1.0e-3f;
    P16(INIT)
#undef INIT
    float vb = 0.999f + seed * 1e-9f, vc = 1.0e-6f * seed;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (KIND == kFmacVV) {
#define OP(i) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a##i) : "v"(vb), "v"(vc));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kMulVV) {
#define OP(i) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(a##i) : "v"(vb));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kFmaVop3) {
#define OP(i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a##i) : "v"(vb), "v"(vc));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kFmacSV) {
#define OP(i) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a##i) : "s"(sb), "v"(vc));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kExp) {
#define OP(i) asm volatile("v_exp_f32 %0, %1" : "+v"(a##i) : "v"(vb));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kPermSwap16) {
            // pairs (a0,a1) .. (a14,a15): each pair is written again 8 instructions later
#define OP2(i, j) asm volatile("v_permlane16_swap_b32 %0, %1" : "+v"(a##i), "+v"(a##j));
#define PS OP2(0, 1) OP2(2, 3) OP2(4, 5) OP2(6, 7) OP2(8, 9) OP2(10, 11) OP2(12, 13) OP2(14, 15)
            PS PS PS PS PS PS PS PS
#undef PS
#undef OP2
        } else if constexpr (KIND == kCndmask) {
#define OP(i) asm volatile("v_cndmask_b32 %0, %0, %1, vcc" : "+v"(a##i) : "v"(vb));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kCndmaskS) {
            const uint64_t cond = (uint64_t)(uint32_t)sb * 0x100000001ull;
#define OP(i) asm volatile("v_cndmask_b32_e64 %0, %0, %1, %2" : "+v"(a##i) : "v"(vb), "s"(cond));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kBfi) {
            const uint32_t vm = (lane & 8) ? 0xffffffffu : 0u;
#define OP(i) asm volatile("v_bfi_b32 %0, %1, %2, %0" : "+v"(a##i) : "v"(vm), "v"(vb));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kCmpCnd) {
            const int vl = lane & 7;
#define OP(i) asm volatile("v_cmp_lt_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, 0, %0, vcc" : "+v"(a##i) : "v"(vl), "v"(i & 3) : "vcc");
            P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kAddDpp) {
#define OP(i) asm volatile("v_add_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(a##i));
            P16(OP) P16(OP) P16(OP) P16(OP)
#undef OP
        } else if constexpr (KIND == kExpFmac4) {
            // 16 groups of (1 exp + 4 fmac) = 80 instructions
#define OP(i) asm volatile("v_exp_f32 %0, %1" : "+v"(a##i) : "v"(vb)); \
            asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a0) : "v"(vb), "v"(vc)); \
            asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a5) : "v"(vb), "v"(vc)); \
            asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a10) : "v"(vb), "v"(vc)); \
            asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a15) : "v"(vb), "v"(vc));
            P16(OP)
#undef OP
        } else {
            // The core: a0,a1 = decay exponents (A*log2e of the two states), a2,a3 = the two
            // states h, a4..a7 = Delta of 4 tokens, a8..a11 = Delta*x of 4 tokens, a12..a15 =
            // (B0, B1, C0, C1) of the token (read from LDS in the kernel). Per token:
            //   e0 = exp2(D*a0); e1 = exp2(D*a1); h0 = e0*h0 + B0*U; h1 = e1*h1 + B1*U;
            //   out = C0*h0 + C1*h1
            // The states alternate between (a2, a3) and (n0, n1) from token to token, as
            // the unrolled kernel's registers do. With KIND == kCoreStruct each decay is one
            // multiply (the next power of a per-token ratio), no exp.
            float e0, e1, n0 = 0.0f, n1 = 0.0f;
#define TOK(DD, UU, H0, H1, N0, N1)                                                      \
    if constexpr (KIND == kCoreMix) {                                                    \
        asm volatile("v_mul_f32 %0, %6, %8\n\tv_exp_f32 %0, %0\n\t"                      \
                     "v_mul_f32 %1, %6, %9\n\tv_exp_f32 %1, %1\n\t"                      \
                     "v_mul_f32 %2, %10, %7\n\tv_fmac_f32 %2, %0, %4\n\t"                \
                     "v_mul_f32 %3, %11, %7\n\tv_fmac_f32 %3, %1, %5\n\t"                \
                     "v_mul_f32 %4, %12, %2\n\tv_fmac_f32 %4, %13, %3"                     \
                     : "=&v"(e0), "=&v"(e1), "=&v"(N0), "=&v"(N1), "+v"(H0), "+v"(H1)      \
                     : "v"(DD), "v"(UU), "v"(a0), "v"(a1), "v"(a12), "v"(a13), "v"(a14),   \
                       "v"(a15));                                                        \
    } else {                                                                             \
        asm volatile("v_mul_f32 %0, %6, %8\n\tv_mul_f32 %1, %0, %9\n\t"                  \
                     "v_mul_f32 %2, %10, %7\n\tv_fmac_f32 %2, %0, %4\n\t"                \
                     "v_mul_f32 %3, %11, %7\n\tv_fmac_f32 %3, %1, %5\n\t"                \
                     "v_mul_f32 %4, %12, %2\n\tv_fmac_f32 %4, %13, %3"                     \
                     : "=&v"(e0), "=&v"(e1), "=&v"(N0), "=&v"(N1), "+v"(H0), "+v"(H1)      \
                     : "v"(DD), "v"(UU), "v"(a0), "v"(a1), "v"(a12), "v"(a13), "v"(a14),   \
                       "v"(a15));                                                        \
    }
            // (the readout goes into the old state's register, H0, which the next token
            // no longer reads: the two state sets alternate)
            TOK(a4, a8, a2, a3, n0, n1) TOK(a5, a9, n0, n1, a2, a3)
            TOK(a6, a10, a2, a3, n0, n1) TOK(a7, a11, n0, n1, a2, a3)
            TOK(a4, a8, a2, a3, n0, n1) TOK(a5, a9, n0, n1, a2, a3)
            TOK(a6, a10, a2, a3, n0, n1) TOK(a7, a11, n0, n1, a2, a3)
#undef TOK
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (lane == 0) {
        uint64_t* r = rec + wave * 6;
        r[0] = t0;
        r[1] = t1;
        r[2] = r0;
        r[3] = r1;
        r[4] = hw;
        r[5] = xcc;
    }
    float s = 0.0f;
#define SUM(i) s += a##i;
    P16(SUM)
#undef SUM
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

inline unsigned grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g > 256 * 32) g = 256 * 32;
    if (g < 1) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" {

// dst[i] = src[i] for i < bytes/16 (bytes a multiple of 16; both 16-byte aligned).
int ssmprobe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const int64_t n = bytes / 16;
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                       (const float4*)src, (float4*)dst, n);
    return (int)hipGetLastError();
}

// Reads src (bytes/16 float4) once; writes out[ssmprobe_read_out_floats(bytes)] partial sums.
int64_t ssmprobe_read_out_floats(int64_t bytes) { return (int64_t)grid_for(bytes / 16) * 256; }
int ssmprobe_read(const void* src, float* out, int64_t bytes, void* stream) {
    const int64_t n = bytes / 16;
    hipLaunchKernelGGL(read_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                       (const float4*)src, out, n);
    return (int)hipGetLastError();
}

int ssmprobe_valu_instr_per_iter(int kind) { return instr_per_iter(kind); }

// nblocks workgroups of 256 threads (4 waves) run `iters` iterations of instruction form
// `kind`. rec: 6 uint64 per wave (memtime start/end, realtime start/end, HW_ID, XCC_ID);
// sink: nblocks*256 floats.
int ssmprobe_valu(int kind, int nblocks, int iters, uint64_t* rec, float* sink, void* stream) {
    const hipStream_t s = (hipStream_t)stream;
    const dim3 g((unsigned)nblocks), b(256);
    switch (kind) {
#define K(N) case N: hipLaunchKernelGGL(valu_kernel<N>, g, b, 0, s, iters, rec, sink, 1.0f, 0x3f7fbe77); break;
        K(0) K(1) K(2) K(3) K(4) K(5) K(6) K(7) K(8) K(9) K(10) K(11) K(12) K(13)
#undef K
        default:
            return -1;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
