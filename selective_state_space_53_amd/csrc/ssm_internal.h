// ssm_internal.h - shared between the C ABI (ssm_abi.cpp) and the kernels
// (ssm_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int kDState = 16;        // states per channel supported by the kernels
constexpr int kTokenTile = 32;     // tokens per scan tile (chunk lengths are multiples)
constexpr int kWaveSegTokens = 512;   // tokens per segment of the wave scan (64 lanes x 8)
// Bytes of the static device scratch behind ssm_scan_fwd_noalloc (one copy per GPU).
constexpr size_t kScratchBytes = size_t(32) << 20;

struct ScanPlan {
    int wavescan = 0;         // 1: the lanes-over-time kernel with the wave prefix combine
                              // (ssm_wavescan.hip; no workspace); 0: the plans below
    int group_channels = 64;  // channels per scan workgroup (32, 48, 64, 80 or 96)
    int64_t ngroups = 0;      // batch * ceil(dim / group_channels)
    int nchunks = 1;        // 1 = single pass
    int64_t chunk_len = 0;  // tokens per chunk (== seqlen for a single pass)
    size_t ws_bcq = 0;      // workspace byte offsets / sizes
    size_t ws_state = 0;
    size_t ws_sum = 0;
    size_t ws_flag = 0;
    size_t ws_total = 0;
};

struct ScanParams {
    const void* x;
    const void* delta;
    const void* z;
    void* y;
    const float* A;
    const float* D;
    const float* bias;
    const float* h0;
    float* h_final;
    float* bcq;          // [batch][8][lpad][4] fp32: B and C widened, per state pair
    float* chunk_state;  // [batch*dim][nchunks][16] (chunked plan) or null
    float* chunk_sum;    // [batch*dim][nchunks]
    int32_t* chunk_flag; // [nchunks]: 1 = a sequence begins inside the chunk (packed input)
    const int32_t* cu;   // packed sequences: [nseq+1] token offsets, or null (batch rows)
    float* ckpt;         // checkpoint pass: [batch][nckpt][dim][16], the state before every
                         // 16th token; null otherwise
    void* q;             // checkpoint pass: [batch][dim][L] io, the output before the gate
                         // (y still gets the gated output), or null
    int64_t nckpt;
    int64_t batch, seqlen, dim, lpad, chunk_len;
    int32_t nchunks, ngroups, groups_per_batch, chunk_offset;
    int32_t nseq;
    int32_t softplus, aligned, reverse, accumulate;
    int32_t structured_a;   // structured A allowed: the wave scan's powers of exp(Delta*A[d,0]),
                            // the sequential lean form's paired decays
};

struct DecodeParams {
    float* state;
    const void* x;
    const void* delta;
    const void* z;
    void* y;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* bias;
    int64_t batch, dim;
    int32_t softplus;
};

struct ConvParams {
    const void* x;          // [rows][seqlen] (decode: [rows])
    const float* w;         // [dim][4]
    const float* bias;      // [dim] or null
    const void* state_in;   // [rows][3] or null (zeros)
    void* y;                // like x
    void* state_out;        // [rows][3] or null; the decode update reads and writes it
    int64_t rows, seqlen, dim;
    int32_t silu, aligned;
};

struct BwdParams {
    const void* x;
    const void* delta;
    const void* z;
    const void* dy;
    const float* A;
    const float* D;
    const float* bias;
    const float* dh_final;   // [batch*dim][16] or null (packed: see below)
    const float* ckpt;       // [batch][nckpt][dim][16]: the state before every 16th token
    const void* q;           // [batch][dim][seqlen] io: the forward output before the gate
    const float* bcq;        // B and C widened, as for the forward
    void* dx;
    void* ddelta;
    void* dz;
    float* dA;               // [dim][16]
    float* dB;               // [batch][seqlen][16]
    float* dC;
    float* dD;               // [dim] or null
    float* dbias;            // [dim] or null
    float* dh0;              // [batch*dim][16] or null
    float* part_bc;          // [batch][groups_per_batch][seqlen][32]: dB (16) then dC (16)
    float* part_A;           // [batch][nchunks][dim][16]
    float* part_D;           // [batch][nchunks][dim]
    float* part_bias;        // [batch][nchunks][dim]
    float* g_carry;          // chunked: [batch*dim][nchunks][16], the gradient reaching the
                             // end of each chunk from later tokens (pass 1: local values)
    float* g_sum;            // chunked: [batch*dim][nchunks], the sum of Delta per chunk
    // packed sequences (batch = 1, seqlen = total tokens): cu_seqlens [nseq+1]; h0,
    // dh_final and dh0 are then per sequence, [nseq][dim][16]; chunk_flag [nchunks]
    // (chunked: 1 where a sequence ends inside the chunk)
    const int32_t* cu;
    const float* h0;
    int32_t* chunk_flag;
    uint32_t* tile_ev;       // [ceil(seqlen/16)]: per 16-token tile, sequence starts (bits
                             // 0..15) and ends (bits 16..31)
    int32_t* tok_seq;        // [seqlen]: the sequence holding each token
    int32_t nseq;
    int64_t batch, seqlen, dim, lpad, nckpt, chunk_len;
    int32_t groups_per_batch, nchunks, chunk_offset, softplus, aligned;
    int32_t reverse;         // 1: the backward of the anti-causal scan (batch rows)
};

// ev_begin / ev_end (may be null) are recorded around the launch of the scan kernel
// that writes y.
hipError_t launch_scan(const ScanPlan& plan, const ScanParams& prm, const void* B, const void* C,
                       bool bf16, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);
// The wave-scan plan: one launch, B and C read directly (ev_begin / ev_end around it).
hipError_t launch_wavescan(const ScanParams& prm, const void* B, const void* C, bool bf16,
                           hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end);
// B and C widened to fp32 into bcq ([batch][8][lpad][4], the scan's layout) on its own:
// the backward runs it when the training forward saved the checkpoints.
hipError_t launch_bc_widen(const void* B, const void* C, float* bcq, int64_t batch,
                           int64_t seqlen, int64_t lpad, bool bf16, hipStream_t stream);
hipError_t launch_state_update(const DecodeParams& prm, bool bf16, hipStream_t stream);
// h_final[i] = h0 ? h0[i] : 0 for i < n (packed input with no tokens: every sequence is empty)
hipError_t launch_copy_state(const float* h0, float* h_final, int64_t n, hipStream_t stream);
// The chunk carry (see carry_kernel): in scan order, chunk_state[c] <- the value carried
// into chunk c; value <- exp(A * sum_c) * value + local_c (just local_c where flag[c]).
hipError_t launch_carry(const float* A, const float* init, float* chunk_state,
                        const float* chunk_sum, const int32_t* chunk_flag, int64_t nrows,
                        int64_t dim, int nchunks, int reverse, hipStream_t stream);
// The backward kernel (ev_begin / ev_end around it) and its reductions.
hipError_t launch_scan_bwd(int cg, const BwdParams& prm, bool bf16, hipStream_t stream,
                           hipEvent_t ev_begin, hipEvent_t ev_end);
// Device address of the static scratch (kScratchBytes) on the device of `stream` (the
// current device for the null stream): looked up once per device, then kept.
hipError_t scratch_address(hipStream_t stream, void** out);
hipError_t launch_conv1d_fwd(const ConvParams& prm, bool bf16, hipStream_t stream);
hipError_t launch_conv1d_update(const ConvParams& prm, bool bf16, hipStream_t stream);

}  // namespace ssm
