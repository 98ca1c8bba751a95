// ssm_kernels.hip - gfx950 kernels of the selective scan and its decode step.
//
// The recurrence (per batch b, channel d, state n, token t):
//   Delta = softplus(delta_raw + bias[d]);  h[n] = exp(Delta*A[d,n])*h[n] + Delta*x*B_t[n]
//   y     = (sum_n C_t[n]*h[n] + D[d]*x) * silu(z)
// State and output equations: "State-Space Models (SSMs) & Mamba" (aidatadrop),
// section "State-Space Models (SSMs): A Resurgent Paradigm for Sequence Modeling".
// Input-dependent B, C, Delta: "Mamba: How Selective State Spaces Achieve 5x
// Faster Inference Than Transformers", section "The selective mechanism".
// Update-then-read and the SiLU gate: "Mamba Architecture Explained", sections
// "The Mamba Innovation: Selective State Updates" and "The Architecture in Practice".
//
// How the work maps onto CDNA4 (the pages' SRAM-tiled CUDA scan, in "The
// convolution trick is gone" of the creativeworksofknowledge Mamba lesson, is prior
// art; what carries over is keeping the state on chip, streaming the sequence once
// and writing back only boundary states):
//
//  * A workgroup owns CG channels of one batch row and all 16 states: CG * 8 threads,
//    i.e. CG / 8 waves (CG a multiple of 16, chosen by the planner's cost model: 16 on
//    the Mamba-130M and 2.8B layer shapes, two waves per workgroup and five workgroups
//    per CU; 32 for the chunked plans of long rows). Each lane keeps one state pair (2
//    states) of one channel in VGPRs for the whole sequence (or chunk); a 16-lane row
//    holds one pair of 16 consecutive channels, a wave four pairs of the same channels.
//  * B_t and C_t do not depend on the channel. A small pass widens them once into
//    fp32 per state pair ([batch][pair][token][B0 B1 C0 C1]); the scan stages each
//    tile's slice through LDS, and a row reads its pair's four values with one
//    row-uniform 16-byte LDS read per token.
//  * The sequence is streamed in tiles of 32 tokens. Per tile: (pre) thread (channel,
//    token quad) computes softplus(Delta), Delta*x, D*x and the gate, and shares Delta
//    and Delta*x through LDS; (core) each lane runs the recurrence over the 32 tokens
//    for its pair and writes the partial readout C*h of the pair to LDS; (post) the
//    8 pairs' partials are summed, D*x added, the gate applied and y stored. Every
//    (t, d) element-wise step is done once, every (t, d, n) step once.
//  * Long sequences with few channel groups are cut into chunks (the tiles-with-
//    final-state idea of the pages' kernel): pass 1 runs each chunk from a zero state
//    and writes only its end state and sum of Delta, a carry pass composes them in
//    chunk order, and pass 2 reruns every chunk from its carried-in state.
//  * The other mapping, lanes over time joined by a wave-wide prefix combine, is in
//    ssm_wavescan.hip.
// No MFMA: there is no dense contraction here; the bound is the VALU (one exp per
// (t, d, n)) with HBM traffic of ~8 bytes per (t, d) in bf16.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

using namespace dev;


// Four consecutive tokens of one row, kept raw in registers between the load
// (issued one tile ahead) and the use. `vec` = the 4 tokens are in range and the
// address is aligned (one 8- or 16-byte load); otherwise `n` (<= 4) valid tokens are
// read one by one and the rest are zero.
template <typename IO> struct Raw4;
template <> struct Raw4<uint16_t> {
    uint32_t w[2];
    __device__ __forceinline__ void load(const uint16_t* p, bool vec, int n) {
        if (vec) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            w[0] = v.x;
            w[1] = v.y;
        } else {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t lo = (2 * k < n) ? p[2 * k] : 0u;
                const uint32_t hi = (2 * k + 1 < n) ? p[2 * k + 1] : 0u;
                w[k] = lo | (hi << 16);
            }
        }
    }
    __device__ __forceinline__ void zero() { w[0] = w[1] = 0u; }
    __device__ __forceinline__ void widen(float* o) const {
        o[0] = bf16_lo(w[0]); o[1] = bf16_hi(w[0]);
        o[2] = bf16_lo(w[1]); o[3] = bf16_hi(w[1]);
    }
};
template <> struct Raw4<float> {
    float v[4];
    __device__ __forceinline__ void load(const float* p, bool vec, int n) {
        if (vec) {
            const float4 a = *reinterpret_cast<const float4*>(p);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = (k < n) ? p[k] : 0.0f;
        }
    }
    __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.0f; }
    __device__ __forceinline__ void widen(float* o) const {
        o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    }
};

template <typename IO> struct Store4;
template <> struct Store4<uint16_t> {
    __device__ __forceinline__ static void store(uint16_t* p, bool vec, int n, const float* v) {
        if (vec) {
            *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]),
                                                      pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (k < n) store_one(p + k, v[k]);
        }
    }
};
template <> struct Store4<float> {
    __device__ __forceinline__ static void store(float* p, bool vec, int n, const float* v) {
        if (vec) {
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (k < n) p[k] = v[k];
        }
    }
};

// ------------------------------------------------------------- B/C widening pass
// bcq[b][p][t][0..3] = (B[b][t][2p], B[b][t][2p+1], C[b][t][2p], C[b][t][2p+1]) in fp32
// for t < seqlen; zero for the padding tokens up to lpad (a multiple of the tile).
// One thread per (b, t, state pair p).
template <typename IO>
__global__ __launch_bounds__(256) void bc_widen_kernel(const IO* __restrict__ B,
                                                       const IO* __restrict__ C,
                                                       float* __restrict__ bcq, int64_t batch,
                                                       int64_t seqlen, int64_t lpad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = batch * lpad * 8;
    if (i >= total) return;
    const int pr = (int)(i & 7);
    const int64_t bt = i >> 3;
    const int64_t b = bt / lpad;
    const int64_t t = bt - b * lpad;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < seqlen) {
        const IO* pb = B + (b * seqlen + t) * kDState + 2 * pr;
        const IO* pc = C + (b * seqlen + t) * kDState + 2 * pr;
        o = make_float4(to_f32(pb[0]), to_f32(pb[1]), to_f32(pc[0]), to_f32(pc[1]));
    }
    *reinterpret_cast<float4*>(bcq + ((b * 8 + pr) * lpad + t) * 4) = o;
}

// --------------------------------------------------------------------- the scan
constexpr int kTile = 32;                 // tokens per tile
constexpr int kLdsRow = kTile + 4;        // padded [channel][token] LDS row (floats)
// Widened B/C of a tile in LDS: [pair][token][B0 B1 C0 C1], each pair's 32 tokens padded
// by 16 bytes. A row reads one 16-byte entry per token, the same for its 16 lanes, and a
// wave's four rows read up to four pairs at once (with 16 channels per workgroup always
// four different ones); unpadded, the pairs are 512 bytes apart and the four reads hit
// the same four banks, padded they fall on four different bank quads.
constexpr int kBcPair = kTile * 4 + 4;    // floats per pair
constexpr int kBcTile = 8 * kBcPair;      // floats of widened B/C per tile (8 state pairs)

// One workgroup = CG channels (a multiple of 16) of one batch row x all 16 states,
// CG*8 threads = CG/8 waves.
//  core mapping: each 16-lane row holds one state pair p (states 2p, 2p+1) of 16
//    consecutive channels; lane = channel. B and C of the row's pair come from LDS
//    with one row-uniform 16-byte read per token.
//  pre/post mapping: thread t = (channel t/8, token quad t%8) of the 32-token tile, so
//    the 8 threads of a channel read and write 64 contiguous bytes (bf16).
// Per tile:
//  pre : widen x, delta, z (loaded one tile earlier), Delta = softplus(delta + bias),
//        u = Delta*x -> LDS; keep D*x and silu(z) for post
//  core: 32 tokens of the recurrence for the lane's (channel, state pair); partial
//        readouts C*h of the pair -> LDS
//  post: sum the 8 pairs' partials, add D*x, gate, store (or add into) y
// LOCAL = pass 1 of the chunked plan: start from zero, write only the chunk's end
// state and its sum of Delta. Otherwise: outputs y (and final states).
// REV = anti-causal: tiles, and tokens inside a tile, are taken from the last to the
// first; the tiles stay where they are in memory, so loads and stores are the same.
// CKPT = a forward that keeps what the backward needs: as the last pass, and it also
// stores, for every 16-token block of the row, the state entering the block in scan
// order (causal: the state before its first token; REV: the state after the token
// that follows it) -- the backward recomputes its tiles from them -- and, when p.q is
// set, the output before the gate.
// PACKED = packed sequences (p.cu set): the state is reset to the sequence's initial state
// before its first token (in the direction of the scan) and saved after its last.
// Those events depend on the token only, so every branch on them is uniform; tiles
// without an event take the same unrolled path as unpacked input.
// LEAN (1: with the gate z, 2: without, 3: with the gate, adding into y -- the second
// direction of a bidirectional scan): the launch guarantees rows of whole aligned tiles
// (seqlen and chunk_len multiples of the tile), every channel of every group in range and
// softplus on: the tile loop then has no per-token selects and no branches around its
// loads and stores, which go through buffer resources (with the per-tile branch below, 8%
// of the kernel's time on the Mamba-2.8B layer shape).
// LEAN 4 (with the gate) and 5 (without), batch rows of a final pass without checkpoints:
// the lean form with structured A. A workgroup whose A rows all satisfy A[d,n] ==
// (n+1) A[d,0] (checked here) takes the odd state's decay of each pair from the even
// one's, exp(Delta A[d,2p+1]) = exp(Delta A[d,2p]) exp(Delta A[d,0]), the second factor
// evaluated once per (token, channel) in the pre stage: one exp per (token, channel,
// pair) instead of two. Other workgroups take the general decays.
template <typename IO, bool LOCAL, bool REV, bool PACKED, bool CKPT, int CG, int LEAN>
__global__ __launch_bounds__(CG * 8) void scan_kernel(const ScanParams p) {
    static_assert(CG % 16 == 0 && CG >= 16 && CG <= 96, "channel group");
    static_assert(!CKPT || !LOCAL, "checkpoints: final pass");
    constexpr bool kLean = LEAN != 0;
    constexpr bool kStructA = LEAN >= 4;
    static_assert(!kStructA || (!LOCAL && !PACKED && !CKPT), "structured A: batch rows, final pass");
    constexpr int kRowsPerPair = CG / 16;
    constexpr bool kOut = !LOCAL;   // this pass writes y (CKPT: also the checkpoints)
    constexpr bool kLeanGate = kOut && (LEAN == 1 || LEAN == 3 || LEAN == 4);
    __shared__ float sD[CG * kLdsRow];
    __shared__ float sU[CG * kLdsRow];
    constexpr int kPStride = CG * kLdsRow;   // floats per pair of partial readouts
    __shared__ float sP[kOut ? 8 * kPStride : 4];
    // One B/C buffer is enough where the next tile's B/C is written after the barrier that
    // ends this tile's core (below); the structured form, whose exp(Delta A[d,0]) row takes
    // the LDS of the second buffer, has one (five 16-channel workgroups per CU still fit).
    constexpr int kBcBufs = kStructA ? 1 : 2;
    __shared__ float sBC[kBcBufs * kBcTile];
    __shared__ float sR[kStructA ? CG * kLdsRow : 1];
    __shared__ int sFlag[1];

    const int tid = threadIdx.x;
    const int g = blockIdx.x % p.ngroups;
    const int c = blockIdx.x / p.ngroups + p.chunk_offset;
    const int64_t b = g / p.groups_per_batch;
    const int64_t d0 = (int64_t)(g % p.groups_per_batch) * CG;
    const int64_t t_beg = (int64_t)c * p.chunk_len;
    const int64_t t_end = (t_beg + p.chunk_len < p.seqlen) ? t_beg + p.chunk_len : p.seqlen;
    const int ntiles = (int)((t_end - t_beg + kTile - 1) / kTile);
    constexpr bool packed = PACKED;   // p.cu is set

    // core mapping: 16-lane row r -> state pair pr, channel block
    const int r = tid >> 4;
    const int pr = r / kRowsPerPair;
    const int cc = (r % kRowsPerPair) * 16 + (tid & 15);      // channel within the group
    const int64_t d = d0 + cc;
    const bool valid = d < p.dim;
    const int64_t row = b * p.dim + d;
    // pre/post mapping: (channel cq, token quad jq)
    const int cq = tid >> 3;
    const int jq = tid & 7;
    const int64_t dq = d0 + cq;
    const bool validq = dq < p.dim;
    const int64_t rowq = b * p.dim + dq;

    float a2[2], h[2];
    bool sall = false;    // structured form: every A row of the workgroup is structured
    float a0q = 0.0f;     // structured form: A[dq,0] log2(e) for the pre stage's channel
    {
        float2 av = make_float2(0.f, 0.f), hv = av;
        if (valid) {
            av = *reinterpret_cast<const float2*>(p.A + d * kDState + 2 * pr);
            if (!LOCAL) {
                if (p.chunk_state)
                    hv = *reinterpret_cast<const float2*>(
                        p.chunk_state + (row * p.nchunks + c) * kDState + 2 * pr);
                else if (p.h0 && !packed)
                    hv = *reinterpret_cast<const float2*>(p.h0 + row * kDState + 2 * pr);
            }
        }
        a2[0] = av.x * kLog2e;
        a2[1] = av.y * kLog2e;
        h[0] = hv.x;
        h[1] = hv.y;
        if constexpr (kStructA) {
            // (every channel of a lean launch is in range) the lane's two states
            const float a0 = p.A[d * kDState];
            const bool ok = av.x == (float)(2 * pr + 1) * a0 && av.y == (float)(2 * pr + 2) * a0;
            if (tid == 0) sFlag[0] = 1;
            __syncthreads();
            if (!ok) sFlag[0] = 0;
            __syncthreads();
            sall = __builtin_amdgcn_readfirstlane(sFlag[0]) != 0;   // uniform
            a0q = p.A[dq * kDState] * kLog2e;
        }
    }
    const float bias = (validq && p.bias) ? p.bias[dq] : 0.0f;
    const float Dd = (validq && p.D) ? p.D[dq] : 0.0f;
    const IO* xr = static_cast<const IO*>(p.x) + rowq * p.seqlen;
    const IO* dr = static_cast<const IO*>(p.delta) + rowq * p.seqlen;
    const IO* zr = (kOut && p.z) ? static_cast<const IO*>(p.z) + rowq * p.seqlen : nullptr;
    IO* yr = kOut ? static_cast<IO*>(p.y) + rowq * p.seqlen : nullptr;
    // CKPT: the state before every 16th token, [batch][t/16][dim][16] (a 16-token block's
    // checkpoints of a workgroup's channels are one contiguous run, which the backward
    // reads whole)
    float* const ck = CKPT ? p.ckpt + (b * p.nckpt * p.dim + d) * kDState + 2 * pr : nullptr;
    const int64_t ckstride = p.dim * kDState;
    // B/C staging: a tile's 256 (pair, token) entries of 16 bytes; the first 256 threads
    // move one each (a 16-channel workgroup has 128 threads: two each)
    constexpr int kMovers = CG * 8 < 256 ? CG * 8 : 256;
    constexpr int kMoves = 256 / kMovers;
    const bool bc_mover = tid < kMovers;
    const float* bcsrc = p.bcq + ((b * 8 + (tid >> 5)) * p.lpad + (tid & 31)) * 4;
    float* const bcdst = sBC + (tid >> 5) * kBcPair + (tid & 31) * 4;
    // LEAN: buffer resources over the workgroup's rows of x, Delta, z, y and q (CG rows of
    // seqlen tokens from row d0) and over its batch row's widened B/C; per lane one byte
    // offset into each (its row and 4 tokens, its B/C entry), per tile one uniform offset
    struct {
        __amdgpu_buffer_rsrc_t x, d, z, y, q, bc;
        uint32_t vo, vbc;
    } lio;
    if constexpr (kLean) {
        const int64_t wb = (b * p.dim + d0) * p.seqlen;
        const uint32_t ext = (uint32_t)(CG * p.seqlen * (int64_t)sizeof(IO));
        lio.x = make_rsrc(static_cast<const IO*>(p.x) + wb, ext);
        lio.d = make_rsrc(static_cast<const IO*>(p.delta) + wb, ext);
        lio.z = make_rsrc(kLeanGate ? static_cast<const IO*>(p.z) + wb : nullptr,
                          kLeanGate ? ext : 0u);
        lio.y = make_rsrc(kOut ? static_cast<const IO*>(p.y) + wb : nullptr, kOut ? ext : 0u);
        lio.q = make_rsrc(CKPT && p.q ? static_cast<const IO*>(p.q) + wb : nullptr,
                          CKPT && p.q ? ext : 0u);
        lio.bc = make_rsrc(p.bcq + b * 8 * p.lpad * 4, (uint32_t)(8 * p.lpad * 16));
        lio.vo = (uint32_t)((cq * p.seqlen + 4 * jq) * (int64_t)sizeof(IO));
        lio.vbc = (uint32_t)((((tid >> 5) & 7) * p.lpad + (tid & 31)) * 16);
    }
    // entry tid + m * kMovers: pair (tid >> 5) + m * kMovers / 32, the same token
    constexpr int64_t kMoveSrc = kMovers / 32;   // pairs per move
    float dsum = 0.0f;

    // ---- packed sequences: s is the sequence of the next token to be scanned, [lo, hi)
    // its tokens. Past the last sequence lo = hi = -1, which matches no token.
    int s = 0;
    int64_t lo = 0, hi = 0;
    bool reset_seen = false;
    // final state of sequence i: the state, or (empty sequence) its initial state
    auto save_final = [&](int i, bool empty) {
        if (LOCAL || !p.h_final || !valid) return;
        float2 v = make_float2(h[0], h[1]);
        if (empty)
            v = p.h0 ? *reinterpret_cast<const float2*>(p.h0 + ((int64_t)i * p.dim + d) * kDState + 2 * pr)
                     : make_float2(0.f, 0.f);
        *reinterpret_cast<float2*>(p.h_final + ((int64_t)i * p.dim + d) * kDState + 2 * pr) = v;
    };
    // step to the next non-empty sequence in scan order, saving the empty ones passed
    auto next_seq = [&]() {
        for (;;) {
            s += REV ? -1 : 1;
            if (s < 0 || s >= p.nseq) {
                lo = hi = -1;
                return;
            }
            lo = p.cu[s];
            hi = p.cu[s + 1];
            if (lo < hi) return;
            save_final(s, true);
        }
    };
    // The tiles this workgroup scans: tbase .. tbase + nt - 1 of the chunk. Pass 1 of packed
    // input needs only the chunk's end state (in scan order), which depends on no token
    // before the last sequence start inside the chunk: the tiles before it are skipped
    // (the reset there replaces whatever state the skipped tokens would have left).
    int tbase = 0, nt = ntiles;
    if (packed && LOCAL) {
        if (!REV) {
            const int64_t st = p.cu[seq_of(p.cu, p.nseq, t_end - 1)];
            if (st > t_beg) {
                tbase = (int)((st - t_beg) / kTile);
                nt = ntiles - tbase;
            }
        } else {
            const int64_t en = p.cu[seq_of(p.cu, p.nseq, t_beg) + 1];
            if (en < t_end) nt = (int)((en - 1 - t_beg) / kTile) + 1;
        }
    }
    if (packed) {
        const int64_t scan_end = t_beg + (int64_t)(tbase + nt) * kTile;
        s = seq_of(p.cu, p.nseq,
                   REV ? (scan_end < t_end ? scan_end : t_end) - 1 : t_beg + (int64_t)tbase * kTile);
        lo = p.cu[s];
        hi = p.cu[s + 1];
        // the workgroup that scans the first token also saves the empty sequences
        // that come before it in scan order
        if (!REV && t_beg == 0)
            for (int i = 0; i < s; ++i) save_final(i, true);
        if (REV && t_end == p.seqlen)
            for (int i = s + 1; i < p.nseq; ++i) save_final(i, true);
    }

    float* const myDq = sD + cq * kLdsRow + 4 * jq;   // pre: this thread's 4 tokens
    float* const myUq = sU + cq * kLdsRow + 4 * jq;
    const float* const coreD = sD + cc * kLdsRow;     // core: the lane's channel
    const float* const coreU = sU + cc * kLdsRow;
    float* const myRq = sR + (kStructA ? cq * kLdsRow + 4 * jq : 0);
    const float* const coreR = sR + (kStructA ? cc * kLdsRow : 0);

    Raw4<IO> rx, rdl, rz;
    float4 rbc[kMoves];
#pragma unroll
    for (int m = 0; m < kMoves; ++m) rbc[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    auto tile_of = [&](int it) { return REV ? tbase + nt - 1 - it : tbase + it; };
    auto load_tile = [&](int ti) {
        const int64_t t0 = t_beg + (int64_t)ti * kTile;
        const int nvalid = (t_end - t0 < kTile) ? (int)(t_end - t0) : kTile;
        const int nq = nvalid - 4 * jq;
        const bool vec = p.aligned && nvalid == kTile;
        // (one uniform branch for the whole tile rather than one per load: the per-load
        // form costs a branch and an exec-mask change per row)
        if constexpr (kLean) {
            const int so = (int)(t0 * (int64_t)sizeof(IO));
            u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(lio.x, (int)lio.vo, so, 0);
            rx.w[0] = v.x;
            rx.w[1] = v.y;
            v = __builtin_amdgcn_raw_buffer_load_b64(lio.d, (int)lio.vo, so, 0);
            rdl.w[0] = v.x;
            rdl.w[1] = v.y;
            if (kLeanGate) {
                v = __builtin_amdgcn_raw_buffer_load_b64(lio.z, (int)lio.vo, so, 0);
                rz.w[0] = v.x;
                rz.w[1] = v.y;
            }
        } else if (vec) {
            if (validq) {
                rx.load(xr + t0 + 4 * jq, true, 4);
                rdl.load(dr + t0 + 4 * jq, true, 4);
                if (zr) rz.load(zr + t0 + 4 * jq, true, 4);
            }
        } else if (validq) {
            rx.load(xr + t0 + 4 * jq, false, nq);
            rdl.load(dr + t0 + 4 * jq, false, nq);
            if (zr) rz.load(zr + t0 + 4 * jq, false, nq);
        }
        if (kLean && bc_mover) {
#pragma unroll
            for (int m = 0; m < kMoves; ++m)
                rbc[m] = __builtin_bit_cast(
                    float4, __builtin_amdgcn_raw_buffer_load_b128(
                                lio.bc, (int)lio.vbc, (int)((m * kMoveSrc * p.lpad + t0) * 16), 0));
        } else if (bc_mover) {
#pragma unroll
            for (int m = 0; m < kMoves; ++m)
                rbc[m] = *reinterpret_cast<const float4*>(bcsrc + (m * kMoveSrc * p.lpad + t0) * 4);
        }
    };
    rx.zero();
    rdl.zero();
    rz.zero();
    load_tile(tile_of(0));
    if (bc_mover) {
#pragma unroll
        for (int m = 0; m < kMoves; ++m)
            *reinterpret_cast<float4*>(bcdst + m * kMoveSrc * kBcPair) = rbc[m];
    }
    wait_vmem();   // nothing in flight at the loop's entry: no wait at its top

    for (int it = 0; it < nt; ++it) {
        const int ti = tile_of(it);
        const int64_t t0 = t_beg + (int64_t)ti * kTile;
        const int nvalid = (t_end - t0 < kTile) ? (int)(t_end - t0) : kTile;
        const int nq = nvalid - 4 * jq;            // valid tokens of this thread's 4 (may be <= 0)
        const bool vec = p.aligned && nvalid == kTile;
        // ---- pre: widen this tile's raw tokens, then start loading the next tile
        float xv[4], dv[4], zv[4];
        rx.widen(xv);
        rdl.widen(dv);
        if (kOut) rz.widen(zv);
        if (it + 1 < nt) load_tile(tile_of(it + 1));
        float dl[4], uu[4], post_a[4], post_g[4];
        // The usual case -- a whole tile, softplus on, a gate if this pass applies one --
        // takes straight-line code; the selects of the general form (padding tokens,
        // options) cost ~2% of the kernel on the Mamba-2.8B layer shape.
        const bool fast = kLean || (vec && p.softplus && (!kOut || zr));
        auto pre = [&](auto fast_c) {
            constexpr bool kFast = decltype(fast_c)::value;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float v = dv[k] + bias;
                float delta = (kFast || p.softplus) ? softplus_f(v) : v;
                if (!kFast) delta = (k < nq) ? delta : 0.0f;   // padding: exp(0) = 1, no input
                dl[k] = delta;
                uu[k] = delta * xv[k];
            }
            if (kOut) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    post_g[k] = (LEAN == 2 || LEAN == 5) ? 1.0f
                                : (kFast || zr)              ? silu_f(zv[k])
                                                             : 1.0f;
                    post_a[k] = Dd * xv[k];
                }
            }
        };
        if (fast) pre(std::true_type{});
        else pre(std::false_type{});
        *reinterpret_cast<float4*>(myDq) = make_float4(dl[0], dl[1], dl[2], dl[3]);
        *reinterpret_cast<float4*>(myUq) = make_float4(uu[0], uu[1], uu[2], uu[3]);
        if (kStructA && sall)   // exp(Delta A[d,0]) of the tile's tokens
            *reinterpret_cast<float4*>(myRq) =
                make_float4(decay_exp2<IO>(dl[0] * a0q), decay_exp2<IO>(dl[1] * a0q),
                            decay_exp2<IO>(dl[2] * a0q), decay_exp2<IO>(dl[3] * a0q));
        __syncthreads();

        // With 32 channels a CU holds several workgroups, out of phase: the core runs at
        // raised wave priority so that the others' load and store phases do not take its
        // issue slots (million-token forward 13.02 -> 12.76 ms, packed 339 -> 335 us in a
        // same-box A/B; with one workgroup per CU, as at 80 channels, it gains nothing)
        if (CG <= 32) __builtin_amdgcn_s_setprio(1);
        // ---- core: the recurrence over the 32 tokens for (channel cc, states 2pr, 2pr+1).
        // Every lane of a row reads the same (B0, B1, C0, C1) of a token from LDS, so B
        // and C arrive in VGPRs and every op below is a plain VOP2 with VGPR operands
        // (the fast FP32 issue path; SGPR or DPP operands halve it).
        const float* bct = sBC + (kBcBufs == 2 ? (it & 1) : 0) * kBcTile + pr * kBcPair;
        float* const pout = sP + pr * kPStride + cc * kLdsRow;
#define SSM_TOKEN(OUT, DS, US, Q)                                                     \
    {                                                                                 \
        const float e0 = decay_exp2<IO>(DS * a2[0]);                                  \
        const float e1 = decay_exp2<IO>(DS * a2[1]);                                  \
        h[0] = __builtin_fmaf(e0, h[0], Q.x * US);                                    \
        h[1] = __builtin_fmaf(e1, h[1], Q.y * US);                                    \
        if (kOut) OUT = __builtin_fmaf(Q.w, h[1], Q.z * h[0]);                        \
        else if (LOCAL && pr == 0) dsum += DS;                                        \
    }
        // the structured form: the odd state's decay from the even one's (RS = exp(Delta
        // A[d,0]) of the token)
#define SSM_TOKEN_S(OUT, DS, US, RS, Q)                                               \
    {                                                                                 \
        const float e0 = decay_exp2<IO>(DS * a2[0]);                                  \
        const float e1 = e0 * RS;                                                     \
        h[0] = __builtin_fmaf(e0, h[0], Q.x * US);                                    \
        h[1] = __builtin_fmaf(e1, h[1], Q.y * US);                                    \
        OUT = __builtin_fmaf(Q.w, h[1], Q.z * h[0]);                                  \
    }
        // quiet tile: no sequence starts or ends inside it (always, for batch rows)
        const int64_t tlast = t0 + nvalid - 1;
        const bool quiet = !packed || (REV ? (hi - 1 != tlast && lo < t0)
                                           : (lo != t0 && hi > tlast + 1));
        if (quiet) {
            // CKPT: the state entering each 16-token block of the tile, in scan order
            // (a block past the end of the row has none)
            auto checkpoint = [&](int64_t blk) {
                if (CKPT && valid && blk * 16 < p.seqlen)
                    *reinterpret_cast<float2*>(ck + blk * ckstride) = make_float2(h[0], h[1]);
            };
            checkpoint(REV ? t0 / 16 + 1 : t0 / 16);
            // the tile in groups of 4 tokens, the LDS operands of a group read one group
            // ahead of their use (S: the structured decays)
            auto groups = [&](auto s_c) {
                constexpr bool S = decltype(s_c)::value;
                float4 nD, nU, nR, n0, n1, n2, n3;
                auto fetch = [&](int tq) {
                    nD = *reinterpret_cast<const float4*>(coreD + tq);
                    nU = *reinterpret_cast<const float4*>(coreU + tq);
                    if (S) nR = *reinterpret_cast<const float4*>(coreR + tq);
                    n0 = *reinterpret_cast<const float4*>(bct + (tq + 0) * 4);
                    n1 = *reinterpret_cast<const float4*>(bct + (tq + 1) * 4);
                    n2 = *reinterpret_cast<const float4*>(bct + (tq + 2) * 4);
                    n3 = *reinterpret_cast<const float4*>(bct + (tq + 3) * 4);
                };
                fetch(REV ? kTile - 4 : 0);
#pragma unroll
                for (int gq = 0; gq < kTile; gq += 4) {
                    const int tq = REV ? kTile - 4 - gq : gq;
                    if (gq == 16) checkpoint(REV ? t0 / 16 : t0 / 16 + 1);
                    const float4 D4 = nD, U4 = nU, q0 = n0, q1 = n1, q2 = n2, q3 = n3;
                    float4 R4;
                    if (S) R4 = nR;
                    if (gq + 4 < kTile) fetch(REV ? kTile - 8 - gq : gq + 4);
                    __builtin_amdgcn_sched_barrier(0);
                    float pp[4];
                    if constexpr (S) {
                        if (!REV) {
                            SSM_TOKEN_S(pp[0], D4.x, U4.x, R4.x, q0)
                            SSM_TOKEN_S(pp[1], D4.y, U4.y, R4.y, q1)
                            SSM_TOKEN_S(pp[2], D4.z, U4.z, R4.z, q2)
                            SSM_TOKEN_S(pp[3], D4.w, U4.w, R4.w, q3)
                        } else {
                            SSM_TOKEN_S(pp[3], D4.w, U4.w, R4.w, q3)
                            SSM_TOKEN_S(pp[2], D4.z, U4.z, R4.z, q2)
                            SSM_TOKEN_S(pp[1], D4.y, U4.y, R4.y, q1)
                            SSM_TOKEN_S(pp[0], D4.x, U4.x, R4.x, q0)
                        }
                    } else if (!REV) {
                        SSM_TOKEN(pp[0], D4.x, U4.x, q0)
                        SSM_TOKEN(pp[1], D4.y, U4.y, q1)
                        SSM_TOKEN(pp[2], D4.z, U4.z, q2)
                        SSM_TOKEN(pp[3], D4.w, U4.w, q3)
                    } else {
                        SSM_TOKEN(pp[3], D4.w, U4.w, q3)
                        SSM_TOKEN(pp[2], D4.z, U4.z, q2)
                        SSM_TOKEN(pp[1], D4.y, U4.y, q1)
                        SSM_TOKEN(pp[0], D4.x, U4.x, q0)
                    }
                    if (kOut)
                        *reinterpret_cast<float4*>(pout + tq) =
                            make_float4(pp[0], pp[1], pp[2], pp[3]);
                }
            };
            if constexpr (kStructA) {
                if (sall) groups(std::true_type{});
                else groups(std::false_type{});
            } else {
                groups(std::false_type{});
            }
        } else {
            // token by token, with the sequence events (padding tokens have none)
            for (int kk = 0; kk < kTile; ++kk) {
                const int k = REV ? kTile - 1 - kk : kk;
                const int64_t t = t0 + k;
                const bool real = k < nvalid;
                // checkpoints: the state entering each 16-token block in scan order, before
                // any reset there (the backward applies the resets itself)
                if (CKPT && valid &&
                    (REV ? ((k == kTile - 1 && nvalid > 16) || k == 15) : (k == 0 || (k == 16 && real))))
                    *reinterpret_cast<float2*>(ck + (t / 16) * ckstride) = make_float2(h[0], h[1]);
                if (real && t == (REV ? hi - 1 : lo)) {     // first token of sequence s
                    float2 hv = make_float2(0.f, 0.f);
                    if (p.h0 && valid)
                        hv = *reinterpret_cast<const float2*>(
                            p.h0 + ((int64_t)s * p.dim + d) * kDState + 2 * pr);
                    h[0] = hv.x;
                    h[1] = hv.y;
                    reset_seen = true;
                }
                const float ds = coreD[k];
                const float us = coreU[k];
                const float4 q = *reinterpret_cast<const float4*>(bct + k * 4);
                float pk = 0.0f;
                SSM_TOKEN(pk, ds, us, q)
                if (kOut) pout[k] = pk;
                if (real && t == (REV ? lo : hi - 1)) {     // last token of sequence s
                    save_final(s, false);
                    next_seq();
                }
            }
        }
#undef SSM_TOKEN
#undef SSM_TOKEN_S
        // pass 1 keeps its results in registers only, so the compiler may sink the whole
        // recurrence below the barrier and then has to hold every LDS operand of the tile
        // at once (~160 VGPRs); an empty asm that claims to update the state keeps the
        // recurrence above it
        if (LOCAL) asm volatile("" : "+v"(h[0]), "+v"(h[1]), "+v"(dsum));
        if (CG <= 32) __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        // the next tile's B/C into the other LDS buffer, or the one buffer (the last
        // readers of either finished before the barrier above; the next ones come after
        // the next barrier). The loads were issued before the core, so the wait is short;
        // taken here, before this tile's stores, it does not wait for them.
        wait_vmem();
        if (bc_mover && it + 1 < nt) {
#pragma unroll
            for (int m = 0; m < kMoves; ++m)
                *reinterpret_cast<float4*>(bcdst + (kBcBufs == 2 ? ((it + 1) & 1) : 0) * kBcTile +
                                           m * kMoveSrc * kBcPair) = rbc[m];
        }

        // ---- post: this thread's 4 tokens: sum the 8 pairs' partials, skip, gate, store
        if (kOut) {
            float yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 a = *reinterpret_cast<const float4*>(sP + q * kPStride + cq * kLdsRow + 4 * jq);
                yv[0] += a.x; yv[1] += a.y; yv[2] += a.z; yv[3] += a.w;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) yv[k] += post_a[k];
            // training forward: q, the output before the gate, for the backward
            if constexpr (kLean) {
                if (CKPT && p.q)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])}, lio.q,
                        (int)lio.vo, (int)(t0 * (int64_t)sizeof(IO)), 0);
            } else if (CKPT && p.q && validq && nq > 0) {
                Store4<IO>::store(static_cast<IO*>(p.q) + rowq * p.seqlen + t0 + 4 * jq, vec, nq,
                                  yv);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) yv[k] *= post_g[k];
            if constexpr (kLean) {
                const int so = (int)(t0 * (int64_t)sizeof(IO));
                if constexpr (LEAN == 3) {
                    const u32x2_t o = __builtin_amdgcn_raw_buffer_load_b64(lio.y, (int)lio.vo, so, 0);
                    yv[0] += bf16_lo(o.x);
                    yv[1] += bf16_hi(o.x);
                    yv[2] += bf16_lo(o.y);
                    yv[3] += bf16_hi(o.y);
                }
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])}, lio.y,
                    (int)lio.vo, so, 0);
            } else if (vec ? validq : (validq && nq > 0)) {
                if (p.accumulate) {
                    Raw4<IO> old;
                    old.load(yr + t0 + 4 * jq, vec, nq);
                    float ov[4];
                    old.widen(ov);
#pragma unroll
                    for (int k = 0; k < 4; ++k) yv[k] += ov[k];
                }
                if (vec) Store4<IO>::store(yr + t0 + 4 * jq, true, 4, yv);
                else Store4<IO>::store(yr + t0 + 4 * jq, false, nq, yv);
            }
        }
    }

    if (LOCAL) {
        if (packed && g == 0 && tid == 0) p.chunk_flag[c] = reset_seen ? 1 : 0;
        if (!valid) return;
        *reinterpret_cast<float2*>(p.chunk_state + (row * p.nchunks + c) * kDState + 2 * pr) =
            make_float2(h[0], h[1]);
        if (pr == 0) p.chunk_sum[row * p.nchunks + c] = dsum;
    } else if (!packed && valid && p.h_final && c == (REV ? 0 : p.nchunks - 1)) {
        *reinterpret_cast<float2*>(p.h_final + row * kDState + 2 * pr) = make_float2(h[0], h[1]);
    }
}

// ------------------------------------------------------------------ chunk carry
// One thread per (row, n). In scan order: the carried-in state of chunk c is written
// over chunk_state[c]; then h <- exp(A*sum_c Delta)*h + local end state of c, or just
// the local end state when a packed sequence begins inside chunk c (the state after
// the chunk then does not depend on what came before it).
__global__ __launch_bounds__(256) void carry_kernel(const float* __restrict__ A,
                                                    const float* __restrict__ h0,
                                                    float* __restrict__ chunk_state,
                                                    const float* __restrict__ chunk_sum,
                                                    const int32_t* __restrict__ chunk_flag,
                                                    int64_t nrows, int64_t dim, int nchunks,
                                                    int reverse) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nrows * kDState) return;
    const int64_t row = i / kDState;
    const int n = (int)(i % kDState);
    const int64_t d = row % dim;
    const float a2 = A[d * kDState + n] * kLog2e;
    float h = (h0 && !chunk_flag) ? h0[row * kDState + n] : 0.0f;
    float* st = chunk_state + row * (int64_t)nchunks * kDState + n;
    const float* sm = chunk_sum + row * (int64_t)nchunks;
    // every chunk but the last in scan order has a local end state and a sum of
    // Delta; the last only receives its carried-in state
    for (int j = 0; j < nchunks - 1; ++j) {
        const int c = reverse ? nchunks - 1 - j : j;
        const float loc = st[(int64_t)c * kDState];
        const float S = sm[c];
        st[(int64_t)c * kDState] = h;
        h = (chunk_flag && chunk_flag[c]) ? loc : __builtin_fmaf(fast_exp2(a2 * S), h, loc);
    }
    st[(int64_t)(reverse ? 0 : nchunks - 1) * kDState] = h;
}

__global__ __launch_bounds__(256) void copy_state_kernel(const float* h0, float* out,
                                                         int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

// ----------------------------------------------------------------- decode step
// Lane = (channel row, state quad j): a wave covers 16 rows x 16 states, i.e. 1 KB of
// contiguous state, read and written with 16-byte accesses. The 4 lanes of a quad
// each evaluate the per-token scalars (cheap next to the state traffic) and reduce
// the readout with two DPP adds. The state is read and written once per token, so
// both go through the streaming (non-temporal) path. Each thread takes two such
// (row, quad) slots half the launch apart and issues the loads of both before using
// either: more bytes in flight per wave (with streaming accesses: 38.2 -> 35.8 us for
// batch 256 x 5120 on gfx950; three or four slots are slower again).
constexpr int kDecodeSlots = 2;
template <typename IO>
__global__ __launch_bounds__(256) void state_update_kernel(const DecodeParams p) {
    constexpr int R = kDecodeSlots;
    const int64_t nslots = p.batch * p.dim * 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;    // a multiple of 4
    const int64_t tid0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int j = (int)(tid0 & 3);
    const IO* xp = static_cast<const IO*>(p.x);
    const IO* dp = static_cast<const IO*>(p.delta);
    float4 hv[R], av[R];
    float xv[R], dv[R], Bv[R][4], Cv[R][4];
    int64_t grow[R], d[R];
    bool ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t tid = tid0 + r * stride;
        ok[r] = tid < nslots;                     // whole quads agree (nslots % 4 == 0)
        grow[r] = ok[r] ? tid >> 2 : 0;           // b * dim + d (row 0 stands in, unused)
        const int64_t b = grow[r] / p.dim;
        d[r] = grow[r] - b * p.dim;
        hv[r] = ok[r] ? load_stream4(p.state + grow[r] * kDState + 4 * j)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
        av[r] = *reinterpret_cast<const float4*>(p.A + d[r] * kDState + 4 * j);
        const IO* Bp = static_cast<const IO*>(p.B) + b * kDState + 4 * j;
        const IO* Cp = static_cast<const IO*>(p.C) + b * kDState + 4 * j;
        xv[r] = to_f32(xp[grow[r]]);
        dv[r] = to_f32(dp[grow[r]]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            Bv[r][k] = to_f32(Bp[k]);
            Cv[r][k] = to_f32(Cp[k]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = dv[r] + (p.bias ? p.bias[d[r]] : 0.0f);
        const float delta = p.softplus ? softplus_f(v) : v;
        const float u = delta * xv[r];
        float hh[4] = {hv[r].x, hv[r].y, hv[r].z, hv[r].w};
        const float aa[4] = {av[r].x, av[r].y, av[r].z, av[r].w};
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hh[k] = __builtin_fmaf(decay_exp2<IO>(delta * aa[k] * kLog2e), hh[k], u * Bv[r][k]);
            acc = __builtin_fmaf(Cv[r][k], hh[k], acc);
        }
        if (ok[r]) store_stream4(p.state + grow[r] * kDState + 4 * j, hh[0], hh[1], hh[2], hh[3]);
        // quad sum: lanes j^1 then j^2 (quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E)
        acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, acc), 0xB1, 0xF, 0xF, false));
        acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, acc), 0x4E, 0xF, 0xF, false));
        if (j == 0 && ok[r]) {
            float s = acc + (p.D ? p.D[d[r]] * xv[r] : 0.0f);
            if (p.z) s *= silu_f(to_f32(static_cast<const IO*>(p.z)[grow[r]]));
            store_one(static_cast<IO*>(p.y) + grow[r], s);
        }
    }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename IO, bool LOCAL, bool REV, bool PACKED, bool CKPT, int LEAN>
hipError_t launch_scan_cg(int cg, dim3 grid, hipStream_t stream, const ScanParams& prm) {
    switch (cg) {
#define SSM_CASE(N)                                                                        \
    case N:                                                                                \
        hipLaunchKernelGGL((scan_kernel<IO, LOCAL, REV, PACKED, CKPT, N, LEAN>), grid,        \
                           dim3(N * 8), 0, stream, prm);                                   \
        break;
        SSM_CASE(16)
        SSM_CASE(32)
        SSM_CASE(48)
        SSM_CASE(64)
        SSM_CASE(80)
        SSM_CASE(96)
#undef SSM_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// the structured-A lean form (16 or 32 channels per workgroup, the groups the planner
// picks where it applies)
template <typename IO, bool REV, int LEAN>
hipError_t launch_scan_cg_sa(int cg, dim3 grid, hipStream_t stream, const ScanParams& prm) {
    if (cg == 16)
        hipLaunchKernelGGL((scan_kernel<IO, false, REV, false, false, 16, LEAN>), grid, dim3(128),
                           0, stream, prm);
    else
        hipLaunchKernelGGL((scan_kernel<IO, false, REV, false, false, 32, LEAN>), grid, dim3(256),
                           0, stream, prm);
    return hipGetLastError();
}

template <typename IO, bool LOCAL, bool REV, bool PACKED, bool CKPT>
hipError_t launch_scan_kernel(int cg, dim3 grid, hipStream_t stream, const ScanParams& prm) {
    // the lean instantiation (bf16): see scan_kernel
    if constexpr (sizeof(IO) == 2) {
        const int64_t tile = kTile;
        // (and 32-bit buffer offsets: a workgroup's rows and a batch row of B/C below 2 GiB)
        if (prm.aligned && prm.softplus && prm.seqlen % tile == 0 &&
            prm.chunk_len % tile == 0 && prm.dim % cg == 0 &&
            (int64_t)cg * prm.seqlen * 2 < (int64_t(1) << 31) && prm.lpad * 128 < (int64_t(1) << 31)) {
            if constexpr (!LOCAL && !PACKED && !CKPT)
                if (prm.structured_a && !prm.accumulate && (cg == 16 || cg == 32))
                    return prm.z ? launch_scan_cg_sa<IO, REV, 4>(cg, grid, stream, prm)
                                 : launch_scan_cg_sa<IO, REV, 5>(cg, grid, stream, prm);
            // Pass 1 of the chunked plan writes no y (the gate and accumulation do not apply);
            // accumulating takes the lean form with the gate and without checkpoints only
            // (the bidirectional use), the general form otherwise.
            if (LOCAL || (!prm.accumulate && prm.z))
                return launch_scan_cg<IO, LOCAL, REV, PACKED, CKPT, 1>(cg, grid, stream, prm);
            if constexpr (!LOCAL) {
                if (!prm.accumulate)
                    return launch_scan_cg<IO, LOCAL, REV, PACKED, CKPT, 2>(cg, grid, stream, prm);
                if constexpr (!CKPT)
                    if (prm.z)
                        return launch_scan_cg<IO, LOCAL, REV, PACKED, CKPT, 3>(cg, grid, stream, prm);
            }
        }
    }
    return launch_scan_cg<IO, LOCAL, REV, PACKED, CKPT, 0>(cg, grid, stream, prm);
}

template <typename IO, bool LOCAL>
hipError_t launch_scan_dir(int cg, dim3 grid, hipStream_t stream, const ScanParams& prm) {
    if (!LOCAL && prm.ckpt) {
        if (prm.cu)
            return prm.reverse
                       ? launch_scan_kernel<IO, false, true, true, true>(cg, grid, stream, prm)
                       : launch_scan_kernel<IO, false, false, true, true>(cg, grid, stream, prm);
        return prm.reverse
                   ? launch_scan_kernel<IO, false, true, false, true>(cg, grid, stream, prm)
                   : launch_scan_kernel<IO, false, false, false, true>(cg, grid, stream, prm);
    }
    if (prm.cu)
        return prm.reverse
                   ? launch_scan_kernel<IO, LOCAL, true, true, false>(cg, grid, stream, prm)
                   : launch_scan_kernel<IO, LOCAL, false, true, false>(cg, grid, stream, prm);
    return prm.reverse ? launch_scan_kernel<IO, LOCAL, true, false, false>(cg, grid, stream, prm)
                       : launch_scan_kernel<IO, LOCAL, false, false, false>(cg, grid, stream, prm);
}

template <typename IO>
hipError_t launch_bc_widen_t(const void* B, const void* C, float* bcq, int64_t batch,
                             int64_t seqlen, int64_t lpad, hipStream_t stream) {
    const int64_t n = batch * lpad * 8;
    hipLaunchKernelGGL(bc_widen_kernel<IO>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream,
                       static_cast<const IO*>(B), static_cast<const IO*>(C), bcq, batch, seqlen,
                       lpad);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_scan_t(const ScanPlan& plan, ScanParams prm, const void* B, const void* C,
                         hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    {
        hipError_t e = launch_bc_widen_t<IO>(B, C, prm.bcq, prm.batch, prm.seqlen, prm.lpad,
                                             stream);
        if (e != hipSuccess) return e;
    }
    const int cg = plan.group_channels;
    if (plan.nchunks == 1) {
        prm.chunk_state = nullptr;
        prm.chunk_offset = 0;
        if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return hipGetLastError();
        hipError_t e = launch_scan_dir<IO, false>(cg, dim3((unsigned)prm.ngroups), stream, prm);
        if (e == hipSuccess && ev1) e = hipEventRecord(ev1, stream);
        return e;
    }
    // pass 1: every chunk but the last in scan order, from a zero state -> end states
    // and sums of Delta (and, for packed input, whether a sequence begins in the chunk)
    {
        ScanParams p1 = prm;
        p1.chunk_offset = prm.reverse ? 1 : 0;
        hipError_t e = launch_scan_dir<IO, true>(
            cg, dim3((unsigned)(prm.ngroups * (int64_t)(plan.nchunks - 1))), stream, p1);
        if (e != hipSuccess) return e;
    }
    {
        const int64_t nrows = prm.batch * prm.dim;
        hipLaunchKernelGGL(carry_kernel, dim3((unsigned)cdiv(nrows * kDState, 256)), dim3(256),
                           0, stream, prm.A, prm.cu ? nullptr : prm.h0, prm.chunk_state,
                           prm.chunk_sum, prm.cu ? prm.chunk_flag : nullptr, nrows, prm.dim,
                           plan.nchunks, prm.reverse);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    prm.chunk_offset = 0;
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return hipGetLastError();
    hipError_t e = launch_scan_dir<IO, false>(
        cg, dim3((unsigned)(prm.ngroups * (int64_t)plan.nchunks)), stream, prm);
    if (e == hipSuccess && ev1) e = hipEventRecord(ev1, stream);
    return e;
}

}  // namespace

hipError_t launch_scan(const ScanPlan& plan, const ScanParams& prm, const void* B, const void* C,
                       bool bf16, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    return bf16 ? launch_scan_t<uint16_t>(plan, prm, B, C, stream, ev_begin, ev_end)
                : launch_scan_t<float>(plan, prm, B, C, stream, ev_begin, ev_end);
}

hipError_t launch_bc_widen(const void* B, const void* C, float* bcq, int64_t batch,
                           int64_t seqlen, int64_t lpad, bool bf16, hipStream_t stream) {
    return bf16 ? launch_bc_widen_t<uint16_t>(B, C, bcq, batch, seqlen, lpad, stream)
                : launch_bc_widen_t<float>(B, C, bcq, batch, seqlen, lpad, stream);
}

hipError_t launch_carry(const float* A, const float* init, float* chunk_state,
                        const float* chunk_sum, const int32_t* chunk_flag, int64_t nrows,
                        int64_t dim, int nchunks, int reverse, hipStream_t stream) {
    hipLaunchKernelGGL(carry_kernel, dim3((unsigned)cdiv(nrows * kDState, 256)), dim3(256), 0,
                       stream, A, init, chunk_state, chunk_sum, chunk_flag, nrows, dim, nchunks,
                       reverse);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* h0, float* h_final, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, h0,
                       h_final, n);
    return hipGetLastError();
}

hipError_t launch_state_update(const DecodeParams& prm, bool bf16, hipStream_t stream) {
    const int64_t slots = prm.batch * prm.dim * 4;
    const dim3 grid((unsigned)cdiv(cdiv(slots, kDecodeSlots), 256));
    if (bf16)
        hipLaunchKernelGGL(state_update_kernel<uint16_t>, grid, dim3(256), 0, stream, prm);
    else
        hipLaunchKernelGGL(state_update_kernel<float>, grid, dim3(256), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace ssm
