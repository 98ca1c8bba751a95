// ssm_bwd.hip - gfx950 kernels of the backward selective scan (training).
//
// The pages say the model trains with parallel scans ("Mamba: Linear-Time Sequence
// Modeling with Selective State Spaces", key points; the aidatadrop page, "The
// Magic of Selective Scan") but never write the gradients down. These kernels
// compute the reverse-mode derivative of the forward recurrence: with
// a_t = exp(Delta_t A), u_t = Delta_t x_t, q_t = sum_n C_t h_t + D x_t and
// G_t = dLoss/dh_t, for t from the last token to the first
//   dq_t = dy_t silu(z_t),   dz_t = dy_t q_t silu'(z_t)
//   G_t  = a_{t+1} G_{t+1} + dq_t C_t
//   dC_t += dq_t h_t,  dB_t += G_t u_t          (summed over channels)
//   dx_t = dq_t D + Delta_t sum_n G_t B_t
//   dDelta_t = x_t sum_n G_t B_t + sum_n G_t h_{t-1} a_t A,  ddelta = dDelta softplus'(v)
//   dA += G_t h_{t-1} a_t Delta_t,  dD += dq_t x_t,  dbias += ddelta,  dh0 = a_0 G_0.
//
// Mapping (the forward's, with 16-token tiles): a workgroup owns CG channels of one
// batch row and all 16 states; a lane keeps 2 states of one channel. The sequence
// is walked tile by tile from the end. Per tile (two barriers):
//   pre    per (channel, 2 tokens): Delta, u, dq into LDS; dz = dy q silu'(z) at once,
//          with q (the output before the gate) written by the forward pass
//   fwd    from the tile's checkpoint (the state before its first token, also written
//          by the forward pass) the 16 states h_t are recomputed into registers
//   bwd    the adjoint recurrence over the 16 tokens (exp recomputed rather than
//          kept): partial G.B and G.h.a.A per state pair -> LDS, dA in registers, and
//          G.u (dB) and dq.h (dC) summed over the 16 channels of a lane row with DPP
//   post   dx, ddelta per (channel, 2 tokens); the workgroup's dB, dC partial sums ->
//          HBM
// Sums over channels across workgroups (dB, dC) and over batch rows (dA, dD, dbias)
// are finished by small reduction kernels in a fixed order: no float atomics, the
// result does not depend on scheduling.
// Variants: REV, the anti-causal scan (time relabelled: tiles and tokens walked the
// other way, h_{t+1} as the state before token t); PACKED, sequences laid end to end
// in one row (per 16-token tile, bit masks of sequence starts and ends from a small
// kernel; tiles with one run token by token and restart the recurrence and its adjoint
// at the boundaries); and the chunked plan (a local pass per chunk, a carry, then
// every chunk from its carried-in gradient).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

// No implicit fusing of a multiply and an add into an FMA in this file: every FMA is
// written out, so a kernel's results do not depend on how the compiler happened to
// schedule or unroll it (the unrolled tile loop would otherwise fuse a few of the adds
// that the rolled loop does not, and change the gradients' last bits).
#pragma clang fp contract(off)

namespace ssm {

namespace {

using namespace dev;

constexpr int kT = 16;            // tokens per backward tile
constexpr int kRowF = kT + 4;     // padded LDS row of the per-channel arrays (floats)
constexpr int kRowP = kT;         // row of the per-pair partial arrays: unpadded (their
                                  // size decides whether two workgroups fit in a CU); the
                                  // 4-token slots of channel c are XOR-swizzled instead
                                  // (swz below)
// widened B/C of a tile: [pair][token][B0 B1 C0 C1], each pair's 16 tokens padded by 16
// bytes, so that the rows of a wave reading two pairs' entries of one token hit different
// banks (unpadded the pairs are 256 bytes apart: the same banks)
constexpr int kBcPairT = kT * 4 + 4;
constexpr int kBcT = 8 * kBcPairT;  // floats of widened B/C per tile

// The swizzle of channel c's 4-token slots in its 64-byte partial row: rows of consecutive
// channels alternate between the two halves of a 128-byte bank line, and bits 1 and 2 of c
// pick four different slots within a half, so 8 consecutive channels writing a 16-byte
// slot each hit 8 distinct bank groups (and 16 of them 16 groups, with 64 banks). With c & 3
// alone, channels c and c + 4 collided: 2.9 -> 1.1 (x 10^7) bank-conflict cycles, about 2%
// of the backward kernel.
__device__ __forceinline__ int swz(int c) { return ((c >> 1) ^ (c >> 2)) & 3; }

// Two consecutive tokens of one row, raw, loaded one tile ahead of their use.
template <typename IO> struct Raw2;
template <> struct Raw2<uint16_t> {
    uint32_t w;
    __device__ __forceinline__ void load(const uint16_t* p, bool vec, int n) {
        if (vec) {
            w = *reinterpret_cast<const uint32_t*>(p);
        } else {
            const uint32_t lo = n > 0 ? p[0] : 0u;
            const uint32_t hi = n > 1 ? p[1] : 0u;
            w = lo | (hi << 16);
        }
    }
    __device__ __forceinline__ void zero() { w = 0u; }
    __device__ __forceinline__ void widen(float* o) const { o[0] = bf16_lo(w); o[1] = bf16_hi(w); }
};
template <> struct Raw2<float> {
    float v[2];
    __device__ __forceinline__ void load(const float* p, bool vec, int n) {
        if (vec) {
            const float2 a = *reinterpret_cast<const float2*>(p);
            v[0] = a.x;
            v[1] = a.y;
        } else {
            v[0] = n > 0 ? p[0] : 0.0f;
            v[1] = n > 1 ? p[1] : 0.0f;
        }
    }
    __device__ __forceinline__ void zero() { v[0] = v[1] = 0.0f; }
    __device__ __forceinline__ void widen(float* o) const { o[0] = v[0]; o[1] = v[1]; }
};

template <typename IO>
__device__ __forceinline__ void store2(IO* p, bool vec, int n, float a, float b) {
    if (vec && sizeof(IO) == 2) {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
    } else if (vec) {
        *reinterpret_cast<float2*>(p) = make_float2(a, b);
    } else {
        if (n > 0) store_one(p, a);
        if (n > 1) store_one(p + 1, b);
    }
}

// DPP lane moves inside a 16-lane row (ctrl is a compile-time constant)
#define SSM_DPP(v, ctrl)                                                                    \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)),   \
                                                          (ctrl), 0xF, 0xF, false))

// Sum four values over the 16 lanes of a row (a reduce-scatter): afterwards lanes 0-3
// hold the sum of v0, lanes 4-7 of v1, lanes 8-11 of v2, lanes 12-15 of v3 (the four
// lanes of a quad the same bits: the last two steps add the same pairs in swapped
// order, and IEEE addition commutes). Each step
// pairs lanes across a half (mirror of the row, then of each half) and moves the
// values the lane does not keep; two quad swaps finish. 6 selects + 5 DPP adds.
__device__ __forceinline__ float row_sum4(float v0, float v1, float v2, float v3, int lane16) {
    const bool lo = lane16 < 8;
    float k0 = lo ? v0 : v2, k1 = lo ? v1 : v3;      // kept: (v0, v1) low, (v2, v3) high
    const float s0 = lo ? v2 : v0, s1 = lo ? v3 : v1;
    k0 += SSM_DPP(s0, 0x140);   // row_mirror: lane i <-> 15 - i
    k1 += SSM_DPP(s1, 0x140);
    const bool lo4 = (lane16 & 4) == 0;
    float k = lo4 ? k0 : k1;
    const float s = lo4 ? k1 : k0;
    k += SSM_DPP(s, 0x141);     // row_half_mirror: lane i <-> 7 - i within each half
    k += SSM_DPP(k, 0x4E);      // quad_perm [2,3,0,1]
    k += SSM_DPP(k, 0xB1);      // quad_perm [1,0,3,2]
    return k;
}

// Packed sequences: the tokens of [t0, t0 + nvalid) (nvalid <= 16) that are the first
// (smask) or last (emask) token of a non-empty sequence, as bit masks over the tile.
__device__ __forceinline__ void tile_events(const int32_t* cu, int nseq, int64_t t0, int nvalid,
                                            uint32_t* smask, uint32_t* emask) {
    uint32_t sm = 0, em = 0;
    const int64_t t1 = t0 + nvalid;
    for (int s = seq_of(cu, nseq, t0); s < nseq; ++s) {   // the sequences overlapping it
        const int64_t st = cu[s], en = cu[s + 1];
        if (st >= t1) break;
        if (en > st) {
            if (st >= t0) sm |= 1u << (uint32_t)(st - t0);
            if (en <= t1) em |= 1u << (uint32_t)(en - 1 - t0);
        }
        if (en >= t1) break;
    }
    *smask = sm;
    *emask = em;
}

// A tile of packed input with sequence boundaries in it, token by token. In scan order
// (REV: from a sequence's last token to its first) the recompute restarts from h0[s] at
// the first token of sequence s; the adjoint, which runs against the scan order, enters
// the last token of s as dh_final[s] (not what the neighbouring sequence carried), takes
// h0[s] as the state before the first token, and writes dh0[s] = a G after it. Otherwise
// the same arithmetic as the quiet path, in the same order per token.
template <int CG, bool REV>
__device__ __forceinline__ void bwd_event_tile(
    const BwdParams& p, int64_t t0, int64_t d, bool valid, int pr, int cc, int lane16,
    uint32_t smask, uint32_t emask, const float* a2, const float* Ar, float hs0, float hs1,
    const float* cD, const float* cU, const float* cQ, const float* bct, float* p1, float* p2,
    float* red, float (&hs)[kT][2], float* Gc, float* dA) {
    constexpr int kLaneRows = CG / 2;
    // the first and last tokens of sequences in scan order
    const uint32_t fmask = REV ? emask : smask, lmask = REV ? smask : emask;
    auto seq_state = [&](const float* base, int s) {   // base[s][d][2pr..2pr+1] or zeros
        float2 v = make_float2(0.f, 0.f);
        if (base && valid)
            v = *reinterpret_cast<const float2*>(base + ((int64_t)s * p.dim + d) * kDState + 2 * pr);
        return v;
    };
    {
        float h0 = hs0, h1 = hs1;
#pragma unroll
        for (int kk = 0; kk < kT; ++kk) {
            const int k = REV ? kT - 1 - kk : kk;
            if (fmask & (1u << k)) {
                const float2 v = seq_state(p.h0, p.tok_seq[t0 + k]);
                h0 = v.x;
                h1 = v.y;
            }
            const float Dk = cD[k], Uk = cU[k];
            const float2 bb = *reinterpret_cast<const float2*>(bct + k * 4);
            h0 = __builtin_fmaf(fast_exp2(Dk * a2[0]), h0, bb.x * Uk);
            h1 = __builtin_fmaf(fast_exp2(Dk * a2[1]), h1, bb.y * Uk);
            hs[k][0] = h0;
            hs[k][1] = h1;
        }
    }
#pragma unroll
    for (int kk = 0; kk < kT; ++kk) {
        const int k = REV ? kk : kT - 1 - kk;
        if (lmask & (1u << k)) {
            const float2 v = seq_state(p.dh_final, p.tok_seq[t0 + k]);
            Gc[0] = v.x;
            Gc[1] = v.y;
        }
        const float Dk = cD[k], Uk = cU[k], Qk = cQ[k];
        const float4 q = *reinterpret_cast<const float4*>(bct + k * 4);
        const float e0 = fast_exp2(Dk * a2[0]);
        const float e1 = fast_exp2(Dk * a2[1]);
        const float G0 = __builtin_fmaf(Qk, q.z, Gc[0]);
        const float G1 = __builtin_fmaf(Qk, q.w, Gc[1]);
        // the state before token k in scan order
        constexpr int kLast = kT - 1;
        float hp0 = REV ? (k < kLast ? hs[k < kLast ? k + 1 : kLast][0] : hs0)
                        : (k > 0 ? hs[k > 0 ? k - 1 : 0][0] : hs0);
        float hp1 = REV ? (k < kLast ? hs[k < kLast ? k + 1 : kLast][1] : hs1)
                        : (k > 0 ? hs[k > 0 ? k - 1 : 0][1] : hs1);
        const bool first = (fmask & (1u << k)) != 0;
        int s = 0;
        if (first) {
            s = p.tok_seq[t0 + k];
            const float2 v = seq_state(p.h0, s);
            hp0 = v.x;
            hp1 = v.y;
        }
        const float o1 = __builtin_fmaf(G1, q.y, G0 * q.x);          // G.B
        Gc[0] = e0 * G0;                                              // a G
        Gc[1] = e1 * G1;
        const float w0 = Gc[0] * hp0;
        const float w1 = Gc[1] * hp1;
        const float o2 = __builtin_fmaf(w1, Ar[1], w0 * Ar[0]);      // G.h.a.A
        dA[0] = __builtin_fmaf(w0, Dk, dA[0]);
        dA[1] = __builtin_fmaf(w1, Dk, dA[1]);
        const float sr = row_sum4(G0 * Uk, G1 * Uk, Qk * hs[k][0], Qk * hs[k][1], lane16);
        red[k * kLaneRows * 4] = sr;
        if (first && p.dh0 && valid)
            *reinterpret_cast<float2*>(p.dh0 + ((int64_t)s * p.dim + d) * kDState + 2 * pr) =
                make_float2(Gc[0], Gc[1]);
        const int slot = (((k >> 2) ^ swz(cc)) << 2) + (k & 3);
        p1[slot] = o1;
        p2[slot] = o2;
        // one scheduling region per token, as the quiet path has one per 4 tokens:
        // hoisting across tokens raises the register count of the whole kernel
        __builtin_amdgcn_sched_barrier(0);
    }
}

// (3 waves per SIMD: the register budget of 168 that lets two workgroups of 48 channels,
// or three of 32, share a CU; 64 channels fill a CU's LDS with one workgroup of 8 waves)
// LEAN: the launch guarantees rows of whole aligned tiles, every channel of every group
// in range, softplus on and a gate: no per-token selects and no branches around the
// loads and stores of the tile loop.
template <typename IO, int CG, bool PACKED, bool REV, bool LEAN = false>
__global__ __launch_bounds__(CG * 8) __attribute__((amdgpu_waves_per_eu(CG == 64 ? 2 : 3)))
void scan_bwd_kernel(const BwdParams p) {
    static_assert(CG % 16 == 0 && CG >= 32 && CG <= 64, "channel group");
    // The adjoint evaluates each token's decays exp(Delta A) again rather than reading back
    // what the recomputation produced: kept in the tile's partial rows in LDS they saved
    // the VALU two exps and two multiplies per token, but since the tile loop lost its
    // per-token selects and branches the LDS is the tighter resource: recomputing is 2%
    // faster (610.4 -> 597.9 us on the 2.8B layer, 22.95 -> 22.61 ms on the million-token
    // row, same box), with the same bits.
    constexpr int kRowsPerPair = CG / 16;
    constexpr int kLaneRows = CG / 2;           // 16-lane rows in the workgroup
    __shared__ float sD[CG * kRowF];            // Delta
    __shared__ float sU[CG * kRowF];            // u = Delta x
    __shared__ float sQ[CG * kRowF];            // dq
    __shared__ float sP1[8 * CG * kRowP];       // per state pair: G.B
    __shared__ float sP2[8 * CG * kRowP];       // per state pair: G.h.a.A
    __shared__ float sBC[2 * kBcT];             // [buffer][pair][token][B0 B1 C0 C1]
    __shared__ float sRed[kT * kLaneRows * 4];  // [token][lane row][dB0 dB1 dC0 dC1]
    __shared__ uint32_t sEv;                    // packed: the tile's event masks

    const int tid = threadIdx.x;
    const int64_t ngroups = p.batch * p.groups_per_batch;
    const int64_t gidx = blockIdx.x % ngroups;
    const int c = (int)(blockIdx.x / ngroups) + p.chunk_offset;   // chunk of the sequence
    const int64_t b = gidx / p.groups_per_batch;
    const int grp = (int)(gidx % p.groups_per_batch);
    const int64_t d0 = (int64_t)grp * CG;
    const int64_t L = p.seqlen;
    const int64_t t_beg = (int64_t)c * p.chunk_len;
    const int64_t t_end = (t_beg + p.chunk_len < L) ? t_beg + p.chunk_len : L;
    const int ntiles = (int)((t_end - t_beg + kT - 1) / kT);

    // core mapping: lane row r holds state pair pr of 16 consecutive channels
    const int r = tid >> 4;
    const int pr = r / kRowsPerPair;
    const int cc = (r % kRowsPerPair) * 16 + (tid & 15);
    const int64_t d = d0 + cc;
    const bool valid = d < p.dim;
    const int64_t row = b * p.dim + d;
    const int lane16 = tid & 15;
    // pre/post mapping: (channel cq, tokens 2jq and 2jq+1 of the tile)
    const int cq = tid >> 3;
    const int jq = tid & 7;
    const int64_t dq = d0 + cq;
    const bool validq = dq < p.dim;
    const int64_t rowq = b * p.dim + dq;

    float a2[2] = {0.f, 0.f}, Ar[2] = {0.f, 0.f}, Gc[2] = {0.f, 0.f}, dA[2] = {0.f, 0.f};
    if (valid) {
        const float2 av = *reinterpret_cast<const float2*>(p.A + d * kDState + 2 * pr);
        Ar[0] = av.x;
        Ar[1] = av.y;
        a2[0] = av.x * kLog2e;
        a2[1] = av.y * kLog2e;
        // the gradient reaching the chunk's last token from later ones (packed: the
        // last token of a sequence takes its dh_final instead, at that token)
        const float* g = p.g_carry ? p.g_carry + (row * p.nchunks + c) * kDState + 2 * pr
                                   : (!PACKED && p.dh_final ? p.dh_final + row * kDState + 2 * pr
                                                            : nullptr);
        if (g) {
            const float2 gv = *reinterpret_cast<const float2*>(g);
            Gc[0] = gv.x;
            Gc[1] = gv.y;
        }
    }
    const float bias = (validq && p.bias) ? p.bias[dq] : 0.0f;
    const float Dd = (validq && p.D) ? p.D[dq] : 0.0f;
    // The eight [batch][dim][L] streams: a base per workgroup (uniform, in SGPRs) and one
    // 32-bit byte offset per lane shared by all eight (the workgroup's CG rows span
    // CG * L * sizeof(IO) < 2^32 bytes; the planner guarantees it). Per-lane 64-bit row
    // pointers would take 16 more VGPRs.
    const int64_t wbase = (b * p.dim + d0) * L;
    const char* xw = reinterpret_cast<const char*>(static_cast<const IO*>(p.x) + wbase);
    const char* dw = reinterpret_cast<const char*>(static_cast<const IO*>(p.delta) + wbase);
    const char* zw =
        p.z ? reinterpret_cast<const char*>(static_cast<const IO*>(p.z) + wbase) : nullptr;
    const char* gw = reinterpret_cast<const char*>(static_cast<const IO*>(p.dy) + wbase);
    const char* qw = reinterpret_cast<const char*>(static_cast<const IO*>(p.q) + wbase);
    char* dxw = reinterpret_cast<char*>(static_cast<IO*>(p.dx) + wbase);
    char* ddw = reinterpret_cast<char*>(static_cast<IO*>(p.ddelta) + wbase);
    char* dzw = p.z ? reinterpret_cast<char*>(static_cast<IO*>(p.dz) + wbase) : nullptr;
    const bool zr = p.z != nullptr;
    const uint32_t lrow = (uint32_t)((int64_t)cq * L * (int64_t)sizeof(IO));
    // byte offset of this thread's 2 tokens starting at token t
    auto at = [&](int64_t t) { return lrow + (uint32_t)((t + 2 * jq) * (int64_t)sizeof(IO)); };
    // checkpoints [batch][L/16][dim][16]: a tile's are one 2 KB run per workgroup, read
    // once, so they are loaded non-temporally and do not push the input rows, which the
    // next tiles read again, out of the L2
    const float* ck = p.ckpt + (b * p.nckpt * p.dim + d) * kDState + 2 * pr;
    const int64_t ckstride = p.dim * kDState;
    float* const pbc = p.part_bc + ((b * p.groups_per_batch + grp) * L) * 32;
    // B/C staging: threads 0..127 move one 16-byte (pair, token) entry per tile
    const bool bc_mover = tid < 128;
    const float* bcsrc = p.bcq + ((b * 8 + (tid >> 4)) * p.lpad + (tid & 15)) * 4;
    float* const bcdst = sBC + (tid >> 4) * kBcPairT + (tid & 15) * 4;
    // LEAN: buffer resources over the workgroup's rows of the eight streams and its batch
    // row's widened B/C; per lane a byte offset into each, per tile a uniform one
    struct {
        __amdgpu_buffer_rsrc_t x, d, z, g, q, dx, dd, dz, bc;
        uint32_t vo, vbc;
    } lio;
    if constexpr (LEAN) {
        const uint32_t ext = (uint32_t)(CG * L * (int64_t)sizeof(IO));
        lio.x = make_rsrc(xw, ext);
        lio.d = make_rsrc(dw, ext);
        lio.z = make_rsrc(zw, ext);
        lio.g = make_rsrc(gw, ext);
        lio.q = make_rsrc(qw, ext);
        lio.dx = make_rsrc(dxw, ext);
        lio.dd = make_rsrc(ddw, ext);
        lio.dz = make_rsrc(dzw, ext);
        lio.bc = make_rsrc(p.bcq + b * 8 * p.lpad * 4, (uint32_t)(8 * p.lpad * 16));
        lio.vo = at(0);
        lio.vbc = (uint32_t)((((tid >> 4) & 7) * p.lpad + (tid & 15)) * 16);
    }

    float* const myD = sD + cq * kRowF + 2 * jq;
    float* const myU = sU + cq * kRowF + 2 * jq;
    float* const myQ = sQ + cq * kRowF + 2 * jq;
    const float* const cD = sD + cc * kRowF;
    const float* const cU = sU + cc * kRowF;
    const float* const cQ = sQ + cc * kRowF;
    float* const p1 = sP1 + (pr * CG + cc) * kRowP;
    float* const p2 = sP2 + (pr * CG + cc) * kRowP;
    // lanes 4j..4j+3 of a row hold its sum of value j (dB0, dB1, dC0, dC1)
    float* const red = sRed + r * 4 + (lane16 >> 2);

    Raw2<IO> rx, rd, rz, rg, rq;
    float4 rbc = make_float4(0.f, 0.f, 0.f, 0.f);
    float2 rck = make_float2(0.f, 0.f);
    // packed: the tile's event masks (starts | ends << 16), loaded by thread 0 with the
    // tile's inputs and passed to the workgroup through LDS. (A uniform load would be
    // moved to a scalar register right away, and the wait for it would also wait for the
    // next tile's prefetched inputs issued before it.)
    uint32_t rev = 0;
    // LEAN batch rows in whole 64-token groups: a 128-byte line of an input row holds the
    // thread's 2 tokens of four consecutive tiles. Loaded tile by tile, a line fetched for
    // one tile was often evicted from the L2 before the next tile's turn (~1.8x the input
    // bytes read); here the first tile of a group loads the four tiles' words at once and
    // holds the later three in `hold` (15 VGPRs), so each line is fetched once. The tile
    // loop is unrolled by the group, so hold[j] stays in fixed registers (moving them
    // along tile by tile cost 3% of the kernel). Not for 48 channels or packed rows: their
    // kernels would spill.
    constexpr bool kGroupLoads = LEAN && !PACKED && CG != 48;
    static_assert(!LEAN || sizeof(IO) == 2, "lean rows are bf16");
    constexpr int kGrp = 4;
    constexpr int kU = kGroupLoads ? kGrp : 1;
    const bool grouped = kGroupLoads && (t_beg % (kGrp * kT)) == 0 && (ntiles % kGrp) == 0;
    uint32_t hold[kGrp - 1][5];
    // the five input rows' words of tile ti (LEAN)
    auto lean_rows = [&](int ti, uint32_t (&w)[5]) {
        const int so = (int)((t_beg + (int64_t)ti * kT) * (int64_t)sizeof(IO));
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(lio.x, (int)lio.vo, so, 0);
        w[1] = __builtin_amdgcn_raw_buffer_load_b32(lio.d, (int)lio.vo, so, 0);
        w[2] = __builtin_amdgcn_raw_buffer_load_b32(lio.z, (int)lio.vo, so, 0);
        w[3] = __builtin_amdgcn_raw_buffer_load_b32(lio.q, (int)lio.vo, so, 0);
        w[4] = __builtin_amdgcn_raw_buffer_load_b32(lio.g, (int)lio.vo, so, 0);
    };
    auto take = [&](const uint32_t (&w)[5]) {
        if constexpr (LEAN) {
            rx.w = w[0];
            rd.w = w[1];
            rz.w = w[2];
            rq.w = w[3];
            rg.w = w[4];
        }
    };
    // ti: tile of the chunk; its checkpoint is the global tile t0 / 16. rows = false: the
    // rows' words come from a group load.
    auto load_tile = [&](int ti, bool rows) {
        const int64_t t0 = t_beg + (int64_t)ti * kT;
        const int nvalid = (t_end - t0 < kT) ? (int)(t_end - t0) : kT;
        const int nq = nvalid - 2 * jq;
        const bool vec = p.aligned && nvalid == kT;
        // one uniform branch for the tile rather than one per load
        if constexpr (LEAN) {
            if (rows) {
                uint32_t w[5];
                lean_rows(ti, w);
                take(w);
            }
        } else if (vec) {
            if (validq) {
                const uint32_t o = at(t0);
                rx.load(reinterpret_cast<const IO*>(xw + o), true, 2);
                rd.load(reinterpret_cast<const IO*>(dw + o), true, 2);
                if (zr) {
                    rz.load(reinterpret_cast<const IO*>(zw + o), true, 2);
                    rq.load(reinterpret_cast<const IO*>(qw + o), true, 2);
                }
                rg.load(reinterpret_cast<const IO*>(gw + o), true, 2);
            }
        } else if (validq) {
            rx.load(reinterpret_cast<const IO*>(xw + at(t0)), false, nq);
            rd.load(reinterpret_cast<const IO*>(dw + at(t0)), false, nq);
            if (zr) {
                rz.load(reinterpret_cast<const IO*>(zw + at(t0)), false, nq);
                rq.load(reinterpret_cast<const IO*>(qw + at(t0)), false, nq);
            }
            rg.load(reinterpret_cast<const IO*>(gw + at(t0)), false, nq);
        }
        if (LEAN && bc_mover)
            rbc = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 lio.bc, (int)lio.vbc, (int)(t0 * 16), 0));
        else if (bc_mover)
            rbc = *reinterpret_cast<const float4*>(bcsrc + t0 * 4);
        if (LEAN || valid) {
            const f32x2_t v = __builtin_nontemporal_load(
                reinterpret_cast<const f32x2_t*>(ck + (t0 / kT) * ckstride));
            rck = make_float2(v.x, v.y);
        }
        if (PACKED && tid == 0) rev = p.tile_ev[t0 / kT];
    };
    rx.zero();
    rd.zero();
    rz.zero();
    rg.zero();
    rq.zero();
    // grouped: tile tn starts a group (the first of its four in the walk's order): its
    // words and the next three tiles' words
    auto load_group = [&](int tn) {
        uint32_t w[5];
        lean_rows(tn, w);
#pragma unroll
        for (int j = 0; j < kGrp - 1; ++j) lean_rows(REV ? tn + 1 + j : tn - 1 - j, hold[j]);
        take(w);
        load_tile(tn, false);
    };
    // the next tile tn, which is the (jj + 1)-th of the current group (grouped, jj <
    // kGrp - 1) or the first of the next group
    auto load_next = [&](int tn, auto jj_c) {
        constexpr int jj = decltype(jj_c)::value;
        if constexpr (kGroupLoads && jj < kGrp - 1) {
            if (grouped) {
                take(hold[jj]);
                load_tile(tn, false);
                return;
            }
        }
        if (grouped) load_group(tn);
        else load_tile(tn, true);
    };
    if (grouped) load_group(REV ? 0 : ntiles - 1);
    else load_tile(REV ? 0 : ntiles - 1, true);

    if (bc_mover) *reinterpret_cast<float4*>(bcdst) = rbc;
    wait_vmem();   // nothing in flight at the loop's entry: no wait at its top

    float dDacc = 0.0f, dbacc = 0.0f;
    for (int it0 = 0; it0 < ntiles; it0 += kU) {
    auto tile_body = [&](auto jj_c) __attribute__((always_inline)) {
        constexpr int jj = decltype(jj_c)::value;
        const int it = it0 + jj;
        const int ti = REV ? it : ntiles - 1 - it;   // the adjoint runs against the scan
        const int64_t t0 = t_beg + (int64_t)ti * kT;
        const int nvalid = (t_end - t0 < kT) ? (int)(t_end - t0) : kT;
        const int nq = nvalid - 2 * jq;
        const bool vec = p.aligned && nvalid == kT;

        // ---- pre: Delta, u, dq to LDS; dz right away (q comes from the forward pass)
        float xv[2], dv[2], zv[2], gv[2], qv[2];
        rx.widen(xv);
        rd.widen(dv);
        rz.widen(zv);
        rg.widen(gv);
        rq.widen(qv);
        // the state entering the tile in scan order (causal: before its first token; REV:
        // after the token that follows it)
        const float hs0 = rck.x, hs1 = rck.y;
        if (PACKED && tid == 0) sEv = rev;
        if (it + 1 < ntiles) load_next(REV ? ti + 1 : ti - 1, jj_c);
        float dl[2], sg[2], dqv[2], uu[2], dzv[2];
        // the usual case (a whole tile, softplus on, a gate) in straight-line code, the
        // general one with its selects for padding tokens and options (bf16 only: with
        // fp32 rows, which take twice the registers, the second copy of the code spills)
        const bool fast = LEAN || (sizeof(IO) == 2 && vec && p.softplus && zr);
        auto pre = [&](auto fast_c) {
            constexpr bool kFast = decltype(fast_c)::value;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float v = dv[k] + bias;
                float delta = (kFast || p.softplus) ? softplus_f(v) : v;
                if (!kFast) delta = k < nq ? delta : 0.0f;   // padding: no decay, no input
                dl[k] = delta;
                sg[k] = (kFast || p.softplus) ? sigmoid_f(v) : 1.0f;
                uu[k] = delta * xv[k];
                const float gz = (kFast || zr) ? silu_f(zv[k]) : 1.0f;
                dqv[k] = gv[k] * gz;
                dzv[k] = (kFast || zr) ? gv[k] * qv[k] * dsilu_f(zv[k]) : 0.0f;
            }
        };
        if (fast) pre(std::true_type{});
        else pre(std::false_type{});
        *reinterpret_cast<float2*>(myD) = make_float2(dl[0], dl[1]);
        *reinterpret_cast<float2*>(myU) = make_float2(uu[0], uu[1]);
        *reinterpret_cast<float2*>(myQ) = make_float2(dqv[0], dqv[1]);
        if constexpr (LEAN) {
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(dzv[0], dzv[1]), lio.dz,
                                                  (int)lio.vo, (int)(t0 * (int64_t)sizeof(IO)), 0);
        } else if (fast) {
            if (validq) store2(reinterpret_cast<IO*>(dzw + at(t0)), true, 2, dzv[0], dzv[1]);
        } else if (zr && validq && nq > 0) {
            store2(reinterpret_cast<IO*>(dzw + at(t0)), vec, nq, dzv[0], dzv[1]);
        }
        __syncthreads();

        // packed: the tile's tokens that start (smask) or end (emask) a sequence; the
        // same for the whole workgroup, so every branch on them is uniform
        const uint32_t ev = PACKED ? sEv : 0u;
        const uint32_t smask = ev & 0xffffu, emask = ev >> 16;
        const float* bct = sBC + (it & 1) * kBcT + pr * kBcPairT;
        // the recomputation and the adjoint (VALU-bound) run at raised wave priority, so
        // that a CU's other workgroups, in their load and store phases, do not take the
        // issue slots from them: 707 -> 674 us on the 2.8B layer, 372 -> 348 us on the
        // 130M layer in a same-box A/B (the same in the forward's core: no gain)
        __builtin_amdgcn_s_setprio(1);
        float hs[kT][2];
        // (tiles with events are the rare case: laid out away from the quiet path)
        if (__builtin_expect(PACKED && (smask | emask) != 0, 0)) {
            bwd_event_tile<CG, REV>(p, t0, d, valid, pr, cc, lane16, smask, emask, a2, Ar, hs0,
                                    hs1, cD, cU, cQ, bct, p1, p2, red, hs, Gc, dA);
        } else {
        // ---- fwd: recompute the 16 states of (channel cc, pair pr) from the checkpoint,
        // in scan order
        {
            float h0 = hs0, h1 = hs1;
#pragma unroll
            for (int gi = 0; gi < kT / 4; ++gi) {
                const int g4 = REV ? kT - 4 - 4 * gi : 4 * gi;
                const float4 D4 = *reinterpret_cast<const float4*>(cD + g4);
                const float4 U4 = *reinterpret_cast<const float4*>(cU + g4);
                const float Ds[4] = {D4.x, D4.y, D4.z, D4.w};
                const float Us[4] = {U4.x, U4.y, U4.z, U4.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = REV ? 3 - jj : jj;
                    const int k = g4 + j;
                    const float2 bb = *reinterpret_cast<const float2*>(bct + k * 4);
                    const float e0 = fast_exp2(Ds[j] * a2[0]);
                    const float e1 = fast_exp2(Ds[j] * a2[1]);
                    h0 = __builtin_fmaf(e0, h0, bb.x * Us[j]);
                    h1 = __builtin_fmaf(e1, h1, bb.y * Us[j]);
                    hs[k][0] = h0;
                    hs[k][1] = h1;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- bwd: the adjoint recurrence over the tile, against the scan order (causal:
        // last token first)
#pragma unroll
        for (int gi = 0; gi < kT / 4; ++gi) {
            const int g4 = REV ? 4 * gi : kT - 4 - 4 * gi;
            const float4 D4 = *reinterpret_cast<const float4*>(cD + g4);
            const float4 U4 = *reinterpret_cast<const float4*>(cU + g4);
            const float4 Q4 = *reinterpret_cast<const float4*>(cQ + g4);
            const float Ds[4] = {D4.x, D4.y, D4.z, D4.w};
            const float Us[4] = {U4.x, U4.y, U4.z, U4.w};
            const float Qs[4] = {Q4.x, Q4.y, Q4.z, Q4.w};
            const int slot = ((g4 >> 2) ^ swz(cc)) << 2;
            float o1[4], o2[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = REV ? jj : 3 - jj;
                const int k = g4 + j;
                const float4 q = *reinterpret_cast<const float4*>(bct + k * 4);
                const float e0 = fast_exp2(Ds[j] * a2[0]);
                const float e1 = fast_exp2(Ds[j] * a2[1]);
                const float G0 = __builtin_fmaf(Qs[j], q.z, Gc[0]);
                const float G1 = __builtin_fmaf(Qs[j], q.w, Gc[1]);
                // the state before token k in scan order
                constexpr int kLast = kT - 1;
                const float hp0 = REV ? (k < kLast ? hs[k < kLast ? k + 1 : kLast][0] : hs0)
                                      : (k > 0 ? hs[k > 0 ? k - 1 : 0][0] : hs0);
                const float hp1 = REV ? (k < kLast ? hs[k < kLast ? k + 1 : kLast][1] : hs1)
                                      : (k > 0 ? hs[k > 0 ? k - 1 : 0][1] : hs1);
                o1[j] = __builtin_fmaf(G1, q.y, G0 * q.x);          // G.B
                // a G: the gradient carried to the token before, and with h_{t-1} the
                // decay terms G h a (2 multiplies fewer per token than G h a on its own;
                // with fp32 inputs, whose prefetched rows take twice the registers, the
                // longer-lived products spill, and the separate form stays)
                float ag0, ag1, w0, w1;
                if constexpr (sizeof(IO) == 2) {
                    ag0 = e0 * G0;
                    ag1 = e1 * G1;
                    w0 = ag0 * hp0;
                    w1 = ag1 * hp1;
                } else {
                    w0 = G0 * hp0 * e0;
                    w1 = G1 * hp1 * e1;
                    ag0 = e0 * G0;
                    ag1 = e1 * G1;
                }
                o2[j] = __builtin_fmaf(w1, Ar[1], w0 * Ar[0]);      // G.h.a.A
                dA[0] = __builtin_fmaf(w0, Ds[j], dA[0]);
                dA[1] = __builtin_fmaf(w1, Ds[j], dA[1]);
                // dB += G u, dC += dq h (this token's state), summed over the row
                const float sr = row_sum4(G0 * Us[j], G1 * Us[j], Qs[j] * hs[k][0],
                                          Qs[j] * hs[k][1], lane16);
                // the 4 lanes of a quad hold the same bits, so all of them write: no
                // branch, and the adjoint stays one scheduling region per 4 tokens
                red[k * kLaneRows * 4] = sr;
                Gc[0] = ag0;
                Gc[1] = ag1;
            }
            *reinterpret_cast<float4*>(p1 + slot) = make_float4(o1[0], o1[1], o1[2], o1[3]);
            *reinterpret_cast<float4*>(p2 + slot) = make_float4(o2[0], o2[1], o2[2], o2[3]);
            // keep the scheduler's hoisting inside the group: across groups it raises the
            // register count past 3 waves per SIMD
            __builtin_amdgcn_sched_barrier(0);
        }
        }   // quiet tile
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        // the next tile's B/C into the other buffer (last read before the barrier above),
        // after a wait for its loads -- issued before the recompute, so short -- taken
        // before this tile's stores, so that it does not wait for them
        wait_vmem();
        if (bc_mover && it + 1 < ntiles)
            *reinterpret_cast<float4*>(bcdst + ((it + 1) & 1) * kBcT) = rbc;

        // ---- post: dx, ddelta for (cq, 2 tokens); the workgroup's dB, dC partial sums
        {
            float2 du = make_float2(0.f, 0.f), da = du;
            const int off = (((jq >> 1) ^ swz(cq)) << 2) + 2 * (jq & 1);   // swizzled slot
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float2 a = *reinterpret_cast<const float2*>(sP1 + (q * CG + cq) * kRowP + off);
                const float2 c = *reinterpret_cast<const float2*>(sP2 + (q * CG + cq) * kRowP + off);
                du.x += a.x;
                du.y += a.y;
                da.x += c.x;
                da.y += c.y;
            }
            const float dus[2] = {du.x, du.y}, das[2] = {da.x, da.y};
            float dxo[2], ddo[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                dxo[k] = __builtin_fmaf(dqv[k], Dd, dus[k] * dl[k]);
                const float dD = __builtin_fmaf(dus[k], xv[k], das[k]);
                ddo[k] = dD * sg[k];
                if (LEAN || vec || k < nq) {
                    dDacc = __builtin_fmaf(dqv[k], xv[k], dDacc);
                    dbacc += ddo[k];
                }
            }
            if constexpr (LEAN) {
                const int so = (int)(t0 * (int64_t)sizeof(IO));
                __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(dxo[0], dxo[1]), lio.dx,
                                                      (int)lio.vo, so, 0);
                __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(ddo[0], ddo[1]), lio.dd,
                                                      (int)lio.vo, so, 0);
            } else if (vec) {
                if (validq) {
                    const uint32_t o = at(t0);
                    store2(reinterpret_cast<IO*>(dxw + o), true, 2, dxo[0], dxo[1]);
                    store2(reinterpret_cast<IO*>(ddw + o), true, 2, ddo[0], ddo[1]);
                }
            } else if (validq && nq > 0) {
                store2(reinterpret_cast<IO*>(dxw + at(t0)), false, nq, dxo[0], dxo[1]);
                store2(reinterpret_cast<IO*>(ddw + at(t0)), false, nq, ddo[0], ddo[1]);
            }
        }
        // 16 tokens x 32 values (dB then dC): value i < 512 (i = tid, tid + CG*8) is the
        // sum over the CG/16 rows of value i & 31 of token i >> 5; a wave writes 64
        // contiguous floats, non-temporally (only the reduction kernel reads them)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = tid + m * CG * 8;
            if (i >= kT * 32) break;
            const int k = i >> 5, v = i & 31;
            const int n = v & 15, which = v >> 4;             // which: 0 = dB, 1 = dC
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < kRowsPerPair; ++j)
                sum += sRed[(k * kLaneRows + (n >> 1) * kRowsPerPair + j) * 4 + which * 2 + (n & 1)];
            if (LEAN || k < nvalid) __builtin_nontemporal_store(sum, &pbc[(t0 + k) * 32 + v]);
        }
    };
        tile_body(std::integral_constant<int, 0>{});
        if constexpr (kU > 1) {
            if (it0 + 1 < ntiles) tile_body(std::integral_constant<int, 1>{});
        }
        if constexpr (kU > 2) {
            if (it0 + 2 < ntiles) tile_body(std::integral_constant<int, 2>{});
            if (it0 + 3 < ntiles) tile_body(std::integral_constant<int, 3>{});
        }
    }

    // ---- per-row results: dh0 = a G at the last token of the scan (the carry after it:
    // causal token 0, REV token L-1), dA partials
    const int64_t prow = (b * p.nchunks + c) * p.dim;   // partials of (batch row, chunk)
    if (valid) {
        if (!PACKED && p.dh0 && c == (REV ? p.nchunks - 1 : 0))
            *reinterpret_cast<float2*>(p.dh0 + row * kDState + 2 * pr) = make_float2(Gc[0], Gc[1]);
        *reinterpret_cast<float2*>(p.part_A + (prow + d) * kDState + 2 * pr) =
            make_float2(dA[0], dA[1]);
    }
    // dD and dbias of channel cq: sum over its 8 token threads (lanes 8c..8c+7)
    dDacc += SSM_DPP(dDacc, 0x141);
    dDacc += SSM_DPP(dDacc, 0x4E);
    dDacc += SSM_DPP(dDacc, 0xB1);
    dbacc += SSM_DPP(dbacc, 0x141);
    dbacc += SSM_DPP(dbacc, 0x4E);
    dbacc += SSM_DPP(dbacc, 0xB1);
    if (jq == 0 && validq) {
        p.part_D[prow + dq] = dDacc;
        p.part_bias[prow + dq] = dbacc;
    }
}

// Pass 1 of the chunked backward: for every chunk but the first in the adjoint's order
// (causal: the last chunk; REV: the first), the gradient the chunk passes on to the
// next token in that order when nothing reaches it from the other side,
//   G_loc = sum over its tokens t of (prod of a_r over the tokens from t to the chunk's
//           edge) dq_t C_t,
// and its sum of Delta (the decay of a gradient crossing the whole chunk is
// exp(A sum Delta)). The same mapping and tiles as the full kernel, only the G chain.
template <typename IO, int CG, bool PACKED, bool REV>
__global__ __launch_bounds__(CG * 8) void scan_bwd_local_kernel(const BwdParams p) {
    static_assert(CG % 16 == 0 && CG >= 32 && CG <= 64, "channel group");
    constexpr int kRowsPerPair = CG / 16;
    __shared__ float sD[CG * kRowF];
    __shared__ float sQ[CG * kRowF];
    __shared__ float sC[8 * kT * 2];            // [pair][token][C0 C1]
    __shared__ uint32_t sEv;                    // packed: the tile's event masks

    const int tid = threadIdx.x;
    const int64_t ngroups = p.batch * p.groups_per_batch;
    const int64_t gidx = blockIdx.x % ngroups;
    const int c = (int)(blockIdx.x / ngroups) + p.chunk_offset;
    const int64_t b = gidx / p.groups_per_batch;
    const int64_t d0 = (int64_t)(gidx % p.groups_per_batch) * CG;
    const int64_t L = p.seqlen;
    const int64_t t_beg = (int64_t)c * p.chunk_len;
    const int64_t t_end = (t_beg + p.chunk_len < L) ? t_beg + p.chunk_len : L;
    const int ntiles = (int)((t_end - t_beg + kT - 1) / kT);
    // packed: the chain restarts from a sequence's dh_final at the sequence's last token
    // in scan order (causal: its last token; REV: its first). Walking against the scan,
    // once the chain reaches such a token of the sequence holding the chunk's far edge
    // (causal: its first token; REV: its last), nothing walked before it matters: start
    // there. The tiles run are tfirst .. tfirst + tcount - 1.
    bool ended = false;   // a sequence's last token in scan order lies inside the chunk
    int tfirst = 0, tcount = ntiles;
    if (PACKED) {
        if (!REV) {
            const int64_t e = (int64_t)p.cu[p.tok_seq[t_beg] + 1] - 1;
            if (e >= t_beg && e < t_end) {
                ended = true;
                tcount = (int)((e - t_beg) / kT) + 1;
            }
        } else {
            const int64_t st = p.cu[p.tok_seq[t_end - 1]];
            if (st >= t_beg && st < t_end) {
                ended = true;
                tfirst = (int)((st - t_beg) / kT);
                tcount = ntiles - tfirst;
            }
        }
    }

    const int r = tid >> 4;
    const int pr = r / kRowsPerPair;
    const int cc = (r % kRowsPerPair) * 16 + (tid & 15);
    const int64_t d = d0 + cc;
    const bool valid = d < p.dim;
    const int64_t row = b * p.dim + d;
    const int cq = tid >> 3;
    const int jq = tid & 7;
    const int64_t dq = d0 + cq;
    const bool validq = dq < p.dim;
    const int64_t rowq = b * p.dim + dq;

    float a2[2] = {0.f, 0.f};
    if (valid) {
        const float2 av = *reinterpret_cast<const float2*>(p.A + d * kDState + 2 * pr);
        a2[0] = av.x * kLog2e;
        a2[1] = av.y * kLog2e;
    }
    const float bias = (validq && p.bias) ? p.bias[dq] : 0.0f;
    const IO* dr = static_cast<const IO*>(p.delta) + rowq * L;
    const IO* zr = p.z ? static_cast<const IO*>(p.z) + rowq * L : nullptr;
    const IO* gr = static_cast<const IO*>(p.dy) + rowq * L;
    float G[2] = {0.f, 0.f}, dsum = 0.0f;
    float* const myD = sD + cq * kRowF + 2 * jq;
    float* const myQ = sQ + cq * kRowF + 2 * jq;
    const float* const cD = sD + cc * kRowF;
    const float* const cQ = sQ + cc * kRowF;
    // a tile's raw inputs, loaded one tile ahead of their use: Delta, z, dy per (channel,
    // 2 tokens) and, for threads 0..127, C of one (state pair, token)
    Raw2<IO> rd, rz, rg;
    float4 rc = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t rev = 0;   // packed: the tile's event masks, via thread 0 and LDS as above
    auto load_tile = [&](int ti) {
        const int64_t t0 = t_beg + (int64_t)ti * kT;
        const int nvalid = (t_end - t0 < kT) ? (int)(t_end - t0) : kT;
        const int nq = nvalid - 2 * jq;
        const bool vec = p.aligned && nvalid == kT;
        rd.zero();
        rz.zero();
        rg.zero();
        if (validq) {
            rd.load(dr + t0 + 2 * jq, vec, nq);
            if (zr) rz.load(zr + t0 + 2 * jq, vec, nq);
            rg.load(gr + t0 + 2 * jq, vec, nq);
        }
        if (tid < 128)
            rc = *reinterpret_cast<const float4*>(
                p.bcq + ((b * 8 + (tid >> 4)) * p.lpad + t0 + (tid & 15)) * 4);
        if (PACKED && tid == 0) rev = p.tile_ev[t0 / kT];
    };
    load_tile(REV ? tfirst : tcount - 1);
    for (int it = 0; it < tcount; ++it) {
        const int ti = REV ? tfirst + it : tcount - 1 - it;
        const int64_t t0 = t_beg + (int64_t)ti * kT;
        const int nvalid = (t_end - t0 < kT) ? (int)(t_end - t0) : kT;
        const int nq = nvalid - 2 * jq;
        float dv[2], zv[2], gv[2];
        rd.widen(dv);
        rz.widen(zv);
        rg.widen(gv);
        const float4 cv4 = rc;
        if (PACKED && tid == 0) sEv = rev;
        if (it + 1 < tcount) load_tile(REV ? ti + 1 : ti - 1);
        // C of the tile, per state pair: threads 0..127 move (pair, token)
        if (tid < 128) *reinterpret_cast<float2*>(sC + tid * 2) = make_float2(cv4.z, cv4.w);
        float dl[2], dqv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float v = dv[k] + bias;
            float delta = p.softplus ? softplus_f(v) : v;
            dl[k] = k < nq ? delta : 0.0f;
            dqv[k] = gv[k] * (zr ? silu_f(zv[k]) : 1.0f);
        }
        *reinterpret_cast<float2*>(myD) = make_float2(dl[0], dl[1]);
        *reinterpret_cast<float2*>(myQ) = make_float2(dqv[0], dqv[1]);
        __syncthreads();
        // packed: the tile's last tokens of sequences in scan order (causal: ends; REV:
        // starts)
        const uint32_t lmask = PACKED ? (REV ? (sEv & 0xffffu) : (sEv >> 16)) : 0u;
        __builtin_amdgcn_s_setprio(1);   // as in the main kernel's recurrences
        const float* ct = sC + pr * kT * 2;
        // packed: at a sequence's last token in scan order the gradient restarts from its
        // dh_final, so the chunk's value no longer depends on what the other chunks carry
#pragma unroll
        for (int kk = 0; kk < kT; ++kk) {
            const int k = REV ? kk : kT - 1 - kk;
            if (PACKED && (lmask & (1u << k))) {
                float2 v = make_float2(0.f, 0.f);
                if (p.dh_final && valid)
                    v = *reinterpret_cast<const float2*>(
                        p.dh_final +
                        ((int64_t)p.tok_seq[t0 + k] * p.dim + d) * kDState + 2 * pr);
                G[0] = v.x;
                G[1] = v.y;
            }
            const float ds = cD[k];
            const float2 cv = *reinterpret_cast<const float2*>(ct + 2 * k);
            const float qk = cQ[k];
            // G_k = dq_k C_k + (what comes from later tokens); then carried to k - 1
            G[0] = fast_exp2(ds * a2[0]) * __builtin_fmaf(qk, cv.x, G[0]);
            G[1] = fast_exp2(ds * a2[1]) * __builtin_fmaf(qk, cv.y, G[1]);
            dsum += ds;
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }
    if (PACKED && gidx == 0 && tid == 0) p.chunk_flag[c] = ended ? 1 : 0;
    if (valid) {
        *reinterpret_cast<float2*>(p.g_carry + (row * p.nchunks + c) * kDState + 2 * pr) =
            make_float2(G[0], G[1]);
        // (packed chunks in which a sequence ends: a partial sum, which the carry ignores)
        if (pr == 0) p.g_sum[row * p.nchunks + c] = dsum;
    }
}

// dB[b][t][n] and dC[b][t][n]: the workgroups' partial sums over channel groups, in
// group order. One thread per (b, t, 32 values).
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part,
                                                            float* __restrict__ dB,
                                                            float* __restrict__ dC,
                                                            int64_t batch, int64_t L,
                                                            int groups) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= batch * L * 32) return;
    const int64_t b = i / (L * 32);
    const int64_t rem = i - b * L * 32;       // t * 32 + n32
    const float* src = part + (b * groups) * L * 32 + rem;
    const int64_t stride = L * 32;
    float s = 0.0f;
    int g = 0;
    // eight loads in flight, added in group order; streaming loads, since every partial is
    // read once (with four plain loads in flight: 38.1 -> 26.8 us on the 2.8B layer's 168 MB)
    for (; g + 8 <= groups; g += 8) {
        float a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = __builtin_nontemporal_load(src + (int64_t)(g + j) * stride);
#pragma unroll
        for (int j = 0; j < 8; ++j) s += a[j];
    }
    for (; g < groups; ++g) s += __builtin_nontemporal_load(src + (int64_t)g * stride);
    const int64_t t = rem / 32;
    const int n32 = (int)(rem % 32);
    float* out = n32 < 16 ? dB : dC;
    out[(b * L + t) * kDState + (n32 & 15)] = s;
}

// dA[d][n], dD[d], dbias[d]: sums over batch rows, in row order.
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(
    const float* __restrict__ part_A, const float* __restrict__ part_D,
    const float* __restrict__ part_bias, float* __restrict__ dA, float* __restrict__ dD,
    float* __restrict__ dbias, int64_t batch, int64_t dim) {
    // batch = the number of partial rows (batch rows x chunks). Eight streaming loads in
    // flight per sum, added in row order: the chunked plans have hundreds of partial rows
    // and few outputs, so the sums are bound by load latency (million-token backward:
    // one thread per (d, n) over 316 chunk rows).
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    auto sum_rows = [&](const float* part, int64_t stride) {
        float s = 0.0f;
        int64_t b = 0;
        for (; b + 8 <= batch; b += 8) {
            float a[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = __builtin_nontemporal_load(part + (b + j) * stride + i);
#pragma unroll
            for (int j = 0; j < 8; ++j) s += a[j];
        }
        for (; b < batch; ++b) s += __builtin_nontemporal_load(part + b * stride + i);
        return s;
    };
    if (i < dim * kDState) dA[i] = sum_rows(part_A, dim * kDState);
    if (i < dim) {
        const float sd = sum_rows(part_D, dim), sb = sum_rows(part_bias, dim);
        if (dD) dD[i] = sd;
        if (dbias) dbias[i] = sb;
    }
}

// Packed input: per 16-token tile of the row, the tokens that start a non-empty sequence
// (bits 0..15) and those that end one (bits 16..31); per token, the sequence holding it
// (the largest s with cu[s] <= t, so never an empty one). One thread per tile.
__global__ __launch_bounds__(256) void bwd_tile_events_kernel(const int32_t* __restrict__ cu,
                                                              int nseq, int64_t L,
                                                              uint32_t* __restrict__ ev,
                                                              int32_t* __restrict__ tok_seq) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t0 = i * kT;
    if (t0 >= L) return;
    const int nvalid = (L - t0 < kT) ? (int)(L - t0) : kT;
    uint32_t sm, em;
    tile_events(cu, nseq, t0, nvalid, &sm, &em);
    ev[i] = sm | (em << 16);
    int s = seq_of(cu, nseq, t0);
    for (int k = 0; k < nvalid; ++k) {
        while (s + 1 < nseq && (int64_t)cu[s + 1] <= t0 + k) ++s;
        tok_seq[t0 + k] = s;
    }
}

// dh0 of the empty packed sequences: their dh_final (or zero); one thread per (s, d, n)
__global__ __launch_bounds__(256) void bwd_empty_seq_kernel(const int32_t* __restrict__ cu,
                                                            int nseq, int64_t dim,
                                                            const float* __restrict__ dh_final,
                                                            float* __restrict__ dh0) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nseq * dim * kDState) return;
    const int s = (int)(i / (dim * kDState));
    if (cu[s] != cu[s + 1]) return;
    dh0[i] = dh_final ? dh_final[i] : 0.0f;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace


hipError_t launch_scan_bwd(int cg, const BwdParams& prm, bool bf16, hipStream_t stream,
                           hipEvent_t ev_begin, hipEvent_t ev_end) {
    const int64_t ngroups = prm.batch * prm.groups_per_batch;
    hipError_t e;
#define SSM_BWD(KERNEL, IO, N, GRID, P)                                                    \
    if (P.cu && P.reverse)                                                                 \
        hipLaunchKernelGGL((KERNEL<IO, N, true, true>), GRID, dim3(N * 8), 0, stream, P);  \
    else if (P.cu)                                                                         \
        hipLaunchKernelGGL((KERNEL<IO, N, true, false>), GRID, dim3(N * 8), 0, stream, P); \
    else if (P.reverse)                                                                    \
        hipLaunchKernelGGL((KERNEL<IO, N, false, true>), GRID, dim3(N * 8), 0, stream, P); \
    else                                                                                   \
        hipLaunchKernelGGL((KERNEL<IO, N, false, false>), GRID, dim3(N * 8), 0, stream, P)
#define SSM_BWD_ALL(KERNEL, GRID, P)                                                       \
    switch (cg * 2 + (bf16 ? 1 : 0)) {                                                     \
        case 65: SSM_BWD(KERNEL, uint16_t, 32, GRID, P); break;                            \
        case 97: SSM_BWD(KERNEL, uint16_t, 48, GRID, P); break;                            \
        case 129: SSM_BWD(KERNEL, uint16_t, 64, GRID, P); break;                           \
        case 64: SSM_BWD(KERNEL, float, 32, GRID, P); break;                               \
        case 96: SSM_BWD(KERNEL, float, 48, GRID, P); break;                               \
        case 128: SSM_BWD(KERNEL, float, 64, GRID, P); break;                              \
        default: return hipErrorInvalidValue;                                              \
    }
    if (prm.cu) {
        hipLaunchKernelGGL(bwd_tile_events_kernel,
                           dim3((unsigned)cdiv(cdiv(prm.seqlen, kT), 256)), dim3(256), 0, stream,
                           prm.cu, prm.nseq, prm.seqlen, prm.tile_ev, prm.tok_seq);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (prm.nchunks > 1) {
        // pass 1: every chunk but the first in the adjoint's order, from a zero gradient;
        // then the carry in that order (causal: from the last chunk backwards), starting
        // from dh_final
        BwdParams p1 = prm;
        p1.chunk_offset = prm.reverse ? 0 : 1;
        const dim3 g1((unsigned)(ngroups * (prm.nchunks - 1)));
        SSM_BWD_ALL(scan_bwd_local_kernel, g1, p1)
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        // (packed: the carry starts from zero and takes a chunk's local value as is where a
        // sequence ends inside it; the last tokens of sequences bring in dh_final)
        e = launch_carry(prm.A, prm.cu ? nullptr : prm.dh_final, prm.g_carry, prm.g_sum,
                         prm.cu ? prm.chunk_flag : nullptr, prm.batch * prm.dim, prm.dim,
                         prm.nchunks, prm.reverse ? 0 : 1, stream);
        if (e != hipSuccess) return e;
    }
    if (ev_begin && hipEventRecord(ev_begin, stream) != hipSuccess) return hipGetLastError();
    {
        BwdParams p2 = prm;
        p2.chunk_offset = 0;
        const dim3 g2((unsigned)(ngroups * prm.nchunks));
        // the lean instantiation (bf16): see scan_bwd_kernel
        // (and a workgroup's rows and a batch row of B/C below 2 GiB, so that every buffer
        // offset is a non-negative 32-bit integer)
        const bool lean = bf16 && prm.aligned && prm.softplus && prm.z &&
                          prm.seqlen % kT == 0 && prm.chunk_len % kT == 0 &&
                          prm.dim % cg == 0 && (int64_t)cg * prm.seqlen * 2 < (int64_t(1) << 31) &&
                          prm.lpad * 128 < (int64_t(1) << 31);
        if (lean) {
            switch (cg) {
#define SSM_LEAN(N)                                                                        \
    case N:                                                                                \
        if (prm.cu && prm.reverse)                                                         \
            hipLaunchKernelGGL((scan_bwd_kernel<uint16_t, N, true, true, true>), g2,          \
                               dim3(N * 8), 0, stream, p2);                                \
        else if (prm.cu)                                                                   \
            hipLaunchKernelGGL((scan_bwd_kernel<uint16_t, N, true, false, true>), g2,         \
                               dim3(N * 8), 0, stream, p2);                                \
        else if (prm.reverse)                                                              \
            hipLaunchKernelGGL((scan_bwd_kernel<uint16_t, N, false, true, true>), g2,         \
                               dim3(N * 8), 0, stream, p2);                                \
        else                                                                               \
            hipLaunchKernelGGL((scan_bwd_kernel<uint16_t, N, false, false, true>), g2,        \
                               dim3(N * 8), 0, stream, p2);                                \
        break;
                SSM_LEAN(32)
                SSM_LEAN(48)
                SSM_LEAN(64)
#undef SSM_LEAN
                default: return hipErrorInvalidValue;
            }
        } else {
            SSM_BWD_ALL(scan_bwd_kernel, g2, p2)
        }
    }
#undef SSM_BWD_ALL
#undef SSM_BWD
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_end && hipEventRecord(ev_end, stream) != hipSuccess) return hipGetLastError();
    {
        const int64_t n = prm.batch * prm.seqlen * 32;
        hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0,
                           stream, prm.part_bc, prm.dB, prm.dC, prm.batch, prm.seqlen,
                           prm.groups_per_batch);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // (64-thread workgroups: a layer's dim x 16 sums spread over every CU)
    hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)cdiv(prm.dim * kDState, 64)),
                       dim3(64), 0, stream, prm.part_A, prm.part_D, prm.part_bias, prm.dA,
                       prm.dD, prm.dbias, prm.batch * prm.nchunks, prm.dim);
    e = hipGetLastError();
    if (e != hipSuccess || !prm.cu || !prm.dh0) return e;
    // packed: an empty sequence's final state is its initial state, so dh0 = dh_final
    const int64_t n = (int64_t)prm.nseq * prm.dim * kDState;
    hipLaunchKernelGGL(bwd_empty_seq_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream,
                       prm.cu, prm.nseq, prm.dim, prm.dh_final, prm.dh0);
    return hipGetLastError();
}

}  // namespace ssm
