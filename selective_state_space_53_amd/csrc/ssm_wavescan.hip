// ssm_wavescan.hip - the selective scan with the time axis spread over the lanes of a
// wavefront, joined by a parallel prefix combine.
//
// The recurrence h_t = a_t h_{t-1} + b_t, with a_t = exp(Delta_t A[d,n]) and
// b_t = Delta_t B_t[n] x_t, is an associative composition of the pairs (a_t, b_t):
//   (a1, b1) then (a2, b2)  =  (a1 a2, a2 b1 + b2),   identity (1, 0).
// The pages name this prefix form as the way Mamba trains in parallel ("Mamba: How
// Selective State Spaces Achieve 5x Faster Inference Than Transformers", section "The
// selective mechanism: input-dependent SSM parameters"; "State-Space Models (SSMs) &
// Mamba", section "Hardware-Aware Parallelism: The Secret Sauce") and describe the tiled
// kernel that keeps the state on chip and writes back only boundary states (the
// creativeworksofknowledge Mamba lesson, section "The convolution trick is gone -- what
// now?"). Here, per (batch, channel) row and state n:
//
//  * A wave owns one row. The sequence is cut into segments of 64 K tokens; lane l owns
//    the K consecutive tokens l K .. l K + K - 1 of the segment (in scan order).
//  * Per segment, once per token: Delta = softplus(delta + bias), u = Delta x (each token
//    by the one lane that owns it, no sharing). Then for each of the 16 states:
//      1. the composite of the lane's K pairs (a_j, b_j): the decays' product taken as
//         one exp of the lane's summed Delta, the inputs folded in order;
//      2. an inclusive scan of the lanes' folds across the 64 lanes (six DPP levels:
//         row_shr 1, 2, 4, 8, then row_bcast 15 and 31), shifted by one lane
//         (wave_shr 1) to the exclusive prefix;
//      3. the state entering the lane = that prefix applied to the state entering the
//         segment (a wave-uniform value, carried in a scalar register);
//      4. the lane's K tokens re-run in order from that state, and the readout
//         y += C_t[n] h_t;
//      5. the state after the segment (lane 63's last token) carried to the next.
//  * Then D x, the SiLU gate, the io-dtype store, and after the last segment h_final.
//
// B_t and C_t are shared by all channels of a batch row: a first small kernel widens them
// once to fp32 in the workspace, laid out per segment as [B or C][state][token] with an
// XOR swizzle of the token index that keeps the lanes' 16-byte LDS reads free of bank
// conflicts; each workgroup (W rows of one batch row) then copies a segment's 64 KB
// straight into LDS (global_load_lds), one segment ahead into a second buffer. No other
// data goes through LDS and the only barrier is the one per segment that hands over the
// staged B/C.
//
// REV = the anti-causal scan: segments are taken from the last to the first and tokens
// inside a segment from the last to the first; the staged B/C and the lanes' registers
// are in scan order, so the combine is the same.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

using namespace dev;

// K consecutive io elements of a row in registers (raw bits), loaded with 16-byte
// accesses when the K tokens are all in range and aligned, else one by one.
template <typename IO, int K> struct RawK;
template <int K> struct RawK<uint16_t, K> {
    static_assert(K % 8 == 0, "bf16 rows are loaded 8 tokens at a time");
    uint32_t w[K / 2];
    __device__ __forceinline__ void load(const uint16_t* p, bool vec, int n) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < K / 8; ++q) {
                const uint4 v = *reinterpret_cast<const uint4*>(p + 8 * q);
                w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < K / 2; ++k) {
                const uint32_t lo = (2 * k < n) ? p[2 * k] : 0u;
                const uint32_t hi = (2 * k + 1 < n) ? p[2 * k + 1] : 0u;
                w[k] = lo | (hi << 16);
            }
        }
    }
    __device__ __forceinline__ float get(int e) const {   // element e in memory order
        return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    }
};
template <int K> struct RawK<float, K> {
    static_assert(K % 4 == 0, "fp32 rows are loaded 4 tokens at a time");
    float v[K];
    __device__ __forceinline__ void load(const float* p, bool vec, int n) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < K / 4; ++q) {
                const float4 a = *reinterpret_cast<const float4*>(p + 4 * q);
                v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = (k < n) ? p[k] : 0.0f;
        }
    }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
};

// K outputs (memory order) stored with 16-byte accesses when vec, else the first n.
template <typename IO, int K> struct StoreK;
template <int K> struct StoreK<uint16_t, K> {
    __device__ __forceinline__ static void store(uint16_t* p, bool vec, int n, const float* o) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < K / 8; ++q)
                *reinterpret_cast<uint4*>(p + 8 * q) =
                    make_uint4(pack_bf16x2(o[8 * q], o[8 * q + 1]), pack_bf16x2(o[8 * q + 2], o[8 * q + 3]),
                               pack_bf16x2(o[8 * q + 4], o[8 * q + 5]),
                               pack_bf16x2(o[8 * q + 6], o[8 * q + 7]));
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (k < n) store_one(p + k, o[k]);
        }
    }
};
template <int K> struct StoreK<float, K> {
    __device__ __forceinline__ static void store(float* p, bool vec, int n, const float* o) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < K / 4; ++q)
                *reinterpret_cast<float4*>(p + 4 * q) =
                    make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (k < n) p[k] = o[k];
        }
    }
};

template <typename V> __device__ __forceinline__ V zero_vec();
template <> __device__ __forceinline__ uint4 zero_vec<uint4>() { return make_uint4(0, 0, 0, 0); }
template <> __device__ __forceinline__ float4 zero_vec<float4>() {
    return make_float4(0.f, 0.f, 0.f, 0.f);
}

// The exclusive prefix, across the 64 lanes of the wave, of the lanes' pairs, for two
// states at once. On entry (a, b) is the lane's own fold; on exit (a, b) is the inclusive
// prefix (lanes 0..l) and (ea, eb) the exclusive one (lanes 0..l-1; lane 0: the identity
// (1, 0)). One level combines this lane's pair with the pair of the lane the DPP control
// selects (earlier tokens): b = b_src a + b, a = a_src a (v_fmac_f32 / v_mul_f32 with a DPP
// source); lanes without a source (row starts for row_shr, rows outside the row mask for
// row_bcast) are not written, which is the identity. Levels: row_shr 1, 2, 4, 8 (inclusive
// inside each 16-lane row), row_bcast 15 to rows 1 and 3, row_bcast 31 to rows 2 and 3,
// then wave_shr 1 for the exclusive prefix. The two states' instructions alternate, so
// every DPP read of a register comes at least two instructions after its write (the
// hazard gfx9-family DPP has); the s_nop 1 at the start covers the writes before the block.
// Needs all 64 lanes active.
__device__ __forceinline__ void wave_scan2(float& a0, float& b0, float& a1, float& b1, float& ea0,
                                           float& eb0, float& ea1, float& eb1) {
#define SSM_LVL(C)                                                              \
    "v_fmac_f32_dpp %1, %1, %0 " C "\n\t"                                      \
    "v_mul_f32_dpp %0, %0, %0 " C "\n\t"                                       \
    "v_fmac_f32_dpp %3, %3, %2 " C "\n\t"                                      \
    "v_mul_f32_dpp %2, %2, %2 " C "\n\t"
    asm volatile(
        "s_nop 1\n\t"
        SSM_LVL("row_shr:1 row_mask:0xf bank_mask:0xf")
        SSM_LVL("row_shr:2 row_mask:0xf bank_mask:0xf")
        SSM_LVL("row_shr:4 row_mask:0xf bank_mask:0xf")
        SSM_LVL("row_shr:8 row_mask:0xf bank_mask:0xf")
        SSM_LVL("row_bcast:15 row_mask:0xa bank_mask:0xf")
        SSM_LVL("row_bcast:31 row_mask:0xc bank_mask:0xf")
        "v_mov_b32 %4, 1.0\n\t"
        "v_mov_b32 %5, 0\n\t"
        "v_mov_b32 %6, 1.0\n\t"
        "v_mov_b32 %7, 0\n\t"
        "v_mov_b32_dpp %4, %0 wave_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %5, %1 wave_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %6, %2 wave_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %7, %3 wave_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "=&v"(ea0), "=&v"(eb0), "=&v"(ea1),
          "=&v"(eb1));
#undef SSM_LVL
}

// Token position inside the staged [state][64 K] rows: bit 2 of the index flipped by bits
// 5 and 6, so that the 16-byte reads of 8 (32 banks) or 16 (64 banks) consecutive lanes at
// a stride of K floats land on distinct banks (K = 8; for K = 4 the plain layout is
// already free of conflicts and the flip keeps it so).
__device__ __forceinline__ int swz(int q) { return q ^ ((((q >> 5) ^ (q >> 6)) & 1) << 2); }

template <typename IO, bool REV, bool STRUCT, int K, int W>
__global__ __launch_bounds__(W * 64) void wavescan_kernel(const ScanParams p) {
    constexpr int T = 64 * K;                 // tokens per segment
    constexpr int SEG_BYTES = 2 * kDState * T * 4;   // the staged B/C of one segment
    constexpr int CHUNKS = SEG_BYTES / 1024;         // 1 KB per wave-wide 16-byte load
    static_assert(CHUNKS % W == 0, "staging chunks per wave");
    __shared__ float sBC[2][2][kDState][T];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gpb = p.groups_per_batch;
    const int64_t b = blockIdx.x / gpb;
    const int64_t d = (int64_t)(blockIdx.x % gpb) * W + w;
    const bool valid = d < p.dim;              // wave-uniform
    const int64_t row = b * p.dim + (valid ? d : 0);
    const int64_t L = p.seqlen;
    const int nseg = (int)((L + T - 1) / T);
    // this batch row's B/C segments, widened to fp32 in the staged layout (wave_bc_kernel)
    const char* bcw = reinterpret_cast<const char*>(p.bcq) + (int64_t)b * nseg * SEG_BYTES;

    // per-row constants (uniform: scalar loads)
    float A2[kDState], hc[kDState];
#pragma unroll
    for (int n = 0; n < kDState; ++n) {
        A2[n] = p.A[(valid ? d : 0) * kDState + n] * kLog2e;
        hc[n] = (p.h0 && valid) ? p.h0[row * kDState + n] : 0.0f;
    }
    // structured A (opt-in): this row's A[n] == (n+1) A[0] exactly, so exp(Delta A[n]) =
    // r^(n+1) with r = exp(Delta A[0]) (wave-uniform; rows that fail take the general path)
    bool row_struct = STRUCT;
    {
        const float a0 = p.A[(valid ? d : 0) * kDState];
#pragma unroll
        for (int n = 1; n < kDState; ++n)
            row_struct = row_struct && (p.A[(valid ? d : 0) * kDState + n] == (float)(n + 1) * a0);
    }
    const float bias = (p.bias && valid) ? p.bias[d] : 0.0f;
    const float Dd = (p.D && valid) ? p.D[d] : 0.0f;
    const IO* xr = static_cast<const IO*>(p.x) + row * L;
    const IO* dr = static_cast<const IO*>(p.delta) + row * L;
    const IO* zr = p.z ? static_cast<const IO*>(p.z) + row * L : nullptr;
    IO* yr = static_cast<IO*>(p.y) + row * L;

    // segment order and token positions. Scan index q = lane*K + j inside segment s
    // is memory token t = t0(s) + q (causal) or t0(s) + T - 1 - q (REV).
    auto seg_of = [&](int i) { return REV ? nseg - 1 - i : i; };
    // first memory token of lane `ln`'s K tokens in segment s
    auto lane_base = [&](int s, int ln) -> int64_t {
        return (int64_t)s * T + (REV ? T - (ln + 1) * K : ln * K);
    };

    // ---- B/C staging: one segment's 64 KB copied straight from the widened workspace into
    // an LDS buffer by the workgroup's waves (global_load_lds_dwordx4: 1 KB per wave-wide
    // load, no registers); complete once every wave has waited for its vector memory
    // accesses and passed the barrier that follows
    auto stage = [&](int s, int buf) {
        const char* src = bcw + (int64_t)s * SEG_BYTES;
        char* dst = reinterpret_cast<char*>(&sBC[buf][0][0][0]);
#pragma unroll
        for (int k = 0; k < CHUNKS / W; ++k) {
            const int c = k * W + w;
            __builtin_amdgcn_global_load_lds(
                src + c * 1024 + lane * 16,
                (__attribute__((address_space(3))) void*)(dst + c * 1024), 16, 0, 0);
        }
    };

    // ---- this lane's x, delta, z of a segment (raw, one segment ahead)
    constexpr bool kPrefetchRows = sizeof(IO) == 2;
    RawK<IO, K> rx, rd, rz;
    auto row_load = [&](int s) {
        const int64_t m0 = lane_base(s, lane);
        const int n = (int)((L - m0 < K) ? (L - m0 < 0 ? 0 : L - m0) : K);
        const bool vec = p.aligned && n == K;
        rx.load(xr + m0, vec, n);
        rd.load(dr + m0, vec, n);
        if (zr) rz.load(zr + m0, vec, n);
    };

    stage(seg_of(0), 0);
    if (valid) row_load(seg_of(0));
    wait_vmem();
    __syncthreads();

    for (int it = 0; it < nseg; ++it) {
        const int s = seg_of(it);
        const int buf = it & 1;
        const int64_t m0 = lane_base(s, lane);
        const int nmem = (int)((L - m0 < K) ? (L - m0 < 0 ? 0 : L - m0) : K);  // valid tokens
        const bool vec = p.aligned && nmem == K;
        if (it + 1 < nseg) stage(seg_of(it + 1), buf ^ 1);
        if (!kPrefetchRows && valid && it > 0) row_load(s);
        // the segment's compute for this wave's row, on the general or the structured path
        auto segment = [&](auto path) {
            constexpr bool S = decltype(path)::value;
            // per token, in scan order j (memory element e = j, or K-1-j for REV)
            float dl[K], u[K];
            float dsum = 0.0f;   // the lane's sum of Delta: its total decay is exp(A dsum)
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const int e = REV ? K - 1 - j : j;
                const float v = rd.get(e) + bias;
                float delta = p.softplus ? softplus_f(v) : v;
                delta = (e < nmem) ? delta : 0.0f;   // padding tokens: (1, 0), the identity
                dl[j] = delta;
                u[j] = delta * rx.get(e);
                dsum += delta;
            }
            // the raw x and z of this segment stay for the epilogue; with bf16 rows the next
            // segment's rows are loaded now into the other set (with fp32 rows, twice the
            // registers, they are loaded at the top of the next segment instead)
            RawK<IO, K> cx = rx, cz = rz;
            if (kPrefetchRows && it + 1 < nseg) row_load(seg_of(it + 1));
            float y[K];
#pragma unroll
            for (int j = 0; j < K; ++j) y[j] = 0.0f;
            // structured rows: per token r = exp(Delta A[0]), per lane R = exp(dsum A[0]);
            // pw / fpw hold the current powers (r^(n+1), R^(n+1)) from state to state
            float rt[K], pw[K], Rt = 0.0f, fpw = 0.0f;
            if constexpr (S) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    rt[j] = decay_exp2<IO>(dl[j] * A2[0]);
                    pw[j] = 0.0f;
                }
                Rt = decay_exp2<IO>(dsum * A2[0]);
            }
            const int lq = lane * K;
            const int m = ((lane >> 2) ^ (lane >> 3)) & 1;   // swz(lq + 4g) = (lq + 4g) ^ (m << 2)
            // two states at a time: their folds, scans and fix-ups interleave
#pragma unroll
            for (int n = 0; n < kDState; n += 2) {
                float a[2][K], bb[2][K], fa[2], fb[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const float* Bn = &sBC[buf][0][n + r][0];
                    float Bv[K];
#pragma unroll
                    for (int g = 0; g < K / 4; ++g) {
                        const float4 bq = *reinterpret_cast<const float4*>(Bn + ((lq + 4 * g) ^ (m << 2)));
                        Bv[4 * g] = bq.x; Bv[4 * g + 1] = bq.y; Bv[4 * g + 2] = bq.z; Bv[4 * g + 3] = bq.w;
                    }
                    // 1. the lane's pairs, and their composite: the decay product as one
                    // exp of the summed Delta, the input folded in order. Structured rows:
                    // the decays and their product are the next powers of r and of R.
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        if constexpr (S) {
                            a[r][j] = (n + r == 0) ? rt[j] : pw[j] * rt[j];
                            pw[j] = a[r][j];
                        } else {
                            a[r][j] = decay_exp2<IO>(dl[j] * A2[n + r]);
                        }
                        bb[r][j] = u[j] * Bv[j];
                    }
                    float f = bb[r][0];
#pragma unroll
                    for (int j = 1; j < K; ++j) f = __builtin_fmaf(a[r][j], f, bb[r][j]);
                    fb[r] = f;
                    if constexpr (S) {
                        fa[r] = (n + r == 0) ? Rt : fpw * Rt;
                        fpw = fa[r];
                    } else {
                        fa[r] = decay_exp2<IO>(dsum * A2[n + r]);
                    }
                }
                // C of the pair, read now so that the scan hides the LDS latency
                float Cv[2][K];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const float* Cn = &sBC[buf][1][n + r][0];
#pragma unroll
                    for (int g = 0; g < K / 4; ++g) {
                        const float4 cq = *reinterpret_cast<const float4*>(Cn + ((lq + 4 * g) ^ (m << 2)));
                        Cv[r][4 * g] = cq.x; Cv[r][4 * g + 1] = cq.y;
                        Cv[r][4 * g + 2] = cq.z; Cv[r][4 * g + 3] = cq.w;
                    }
                }
                // 2. the exclusive prefix of the lanes' composites
                float ea0, eb0, ea1, eb1;
                wave_scan2(fa[0], fb[0], fa[1], fb[1], ea0, eb0, ea1, eb1);
                // 3. the state entering this lane's tokens; 4. every token's state, in order,
                // and the readout; 5. the state after the segment (lane 63's last token)
                const float ea[2] = {ea0, ea1}, eb[2] = {eb0, eb1};
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    float h = __builtin_fmaf(ea[r], hc[n + r], eb[r]);
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        h = __builtin_fmaf(a[r][j], h, bb[r][j]);
                        y[j] = __builtin_fmaf(Cv[r][j], h, y[j]);
                    }
                    hc[n + r] = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h), 63));
                }
                // the readout sums are materialized here: otherwise the compiler may sink
                // every state's readout into the epilogue and keep all 16 x K states alive
#pragma unroll
                for (int j = 0; j < K; ++j) asm volatile("" : "+v"(y[j]));
                // keep each pair of states' loads and temporaries to itself
                __builtin_amdgcn_sched_barrier(0);
            }
            // epilogue: skip term, gate, store (memory order)
            float o[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const int e = REV ? K - 1 - j : j;
                const float xe = cx.get(e);
                float v = y[j] + Dd * xe;
                if (zr) v *= silu_f(cz.get(e));
                o[e] = v;
            }
            if (p.accumulate) {
                RawK<IO, K> old;
                old.load(yr + m0, vec, nmem);
#pragma unroll
                for (int e = 0; e < K; ++e) o[e] += old.get(e);
            }
            if (nmem > 0) StoreK<IO, K>::store(yr + m0, vec, nmem, o);
        };
        if (valid) {
            if constexpr (STRUCT) {
                if (row_struct) segment(std::true_type{});
                else segment(std::false_type{});
            } else {
                segment(std::false_type{});
            }
        }
        wait_vmem();   // this wave's part of the next segment's B/C is in LDS
        __syncthreads();
    }
    if (valid && p.h_final && lane == 0) {
        float4* hf = reinterpret_cast<float4*>(p.h_final + row * kDState);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            hf[q] = make_float4(hc[4 * q], hc[4 * q + 1], hc[4 * q + 2], hc[4 * q + 3]);
    }
}

// B and C widened to fp32 into the wave scan's staged layout: per (batch row b, segment s
// of T tokens), [B or C][state n][swz(q)] for the scan-order index q of each token of the
// segment (zeros for the padding tokens past the end), so that staging a segment is one
// contiguous copy. One thread per (b, s, q).
template <typename IO, bool REV, int T>
__global__ __launch_bounds__(256) void wave_bc_kernel(const IO* __restrict__ B,
                                                      const IO* __restrict__ C,
                                                      float* __restrict__ out, int64_t batch,
                                                      int64_t seqlen, int64_t nseg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= batch * nseg * T) return;
    const int q = (int)(i % T);
    const int64_t bs = i / T;                  // b * nseg + s
    const int64_t s = bs % nseg;
    const int64_t b = bs / nseg;
    const int64_t t = s * T + (REV ? T - 1 - q : q);
    float* o = out + bs * (2 * kDState * T) + swz(q);
    if (t < seqlen) {
        const IO* pb = B + (b * seqlen + t) * kDState;
        const IO* pc = C + (b * seqlen + t) * kDState;
#pragma unroll
        for (int n = 0; n < kDState; ++n) {
            o[n * T] = to_f32(pb[n]);
            o[(kDState + n) * T] = to_f32(pc[n]);
        }
    } else {
#pragma unroll
        for (int n = 0; n < 2 * kDState; ++n) o[n * T] = 0.0f;
    }
}

template <typename IO, bool REV>
hipError_t launch_wavescan_t(const ScanParams& prm, const void* B, const void* C,
                             hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int K = 8, W = 16, T = 64 * K;
    static_assert(T == kWaveSegTokens, "segment length of the workspace layout");
    ScanParams p = prm;
    p.groups_per_batch = (int32_t)((p.dim + W - 1) / W);
    const int64_t nseg = (p.seqlen + T - 1) / T;
    const int64_t n = p.batch * nseg * T;
    hipLaunchKernelGGL((wave_bc_kernel<IO, REV, T>), dim3((unsigned)((n + 255) / 256)), dim3(256),
                       0, stream, static_cast<const IO*>(B), static_cast<const IO*>(C), p.bcq,
                       p.batch, p.seqlen, nseg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(p.batch * p.groups_per_batch));
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return hipGetLastError();
    if (p.structured_a)
        hipLaunchKernelGGL((wavescan_kernel<IO, REV, true, K, W>), grid, dim3(W * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((wavescan_kernel<IO, REV, false, K, W>), grid, dim3(W * 64), 0, stream, p);
    e = hipGetLastError();
    if (e == hipSuccess && ev1) e = hipEventRecord(ev1, stream);
    return e;
}

}  // namespace

hipError_t launch_wavescan(const ScanParams& prm, const void* B, const void* C, bool bf16,
                           hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (bf16)
        return prm.reverse
                   ? launch_wavescan_t<uint16_t, true>(prm, B, C, stream, ev_begin, ev_end)
                   : launch_wavescan_t<uint16_t, false>(prm, B, C, stream, ev_begin, ev_end);
    return prm.reverse ? launch_wavescan_t<float, true>(prm, B, C, stream, ev_begin, ev_end)
                       : launch_wavescan_t<float, false>(prm, B, C, stream, ev_begin, ev_end);
}

}  // namespace ssm
