// ssm_abi.cpp - the C ABI of libssmscan: host-side validation, planning and launch.
//
// Every check here runs on the host before anything is enqueued; a failed check
// returns a status and launches nothing. The entry points and their contracts are
// documented in include/ssm_scan.h.

#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ssm_internal.h"

namespace {

thread_local char g_last_error[512] = "";

ssm_status fail(ssm_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

constexpr int64_t kMaxBytes = int64_t(1) << 62;

// a*b*c*d without overflow past kMaxBytes; false when it would.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > kMaxBytes / a) return false;
    *out = a * b;
    return true;
}

bool bytes4(int64_t a, int64_t b, int64_t c, int64_t e, int64_t* out) {
    int64_t t;
    return mul_ok(a, b, &t) && mul_ok(t, c, &t) && mul_ok(t, e, out);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Region {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Region& a, const Region& b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

Region region(const char* name, const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Region{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// LDS bytes of one scan workgroup of cg channels (must match the kernel's arrays):
// Delta, Delta*x and (not in pass 1) the 8 partial readouts, [cg][36] floats each,
// plus two tiles of widened B/C, 8 x (32 x 4 + 4) floats each.
int64_t scan_lds_bytes(int cg, bool local) {
    return (int64_t)((local ? 2 : 10) * cg * 36 + (local ? 4 : 0) + 2 * 8 * 132) * 4;
}

// ---- launch cost model -------------------------------------------------------------
// SIMD cycles per wave per (token, state pair) of the recurrence, by waves resident on
// the SIMD: one wave cannot hide the exp/FMA latencies, more than three add little
// (measured on gfx950 with a probe kernel running the same instruction mix).
double wave_cost(int64_t waves_per_simd) {
    static const double kCost[] = {0.0, 55.5, 36.5, 31.0, 30.7};
    return waves_per_simd <= 4 ? kCost[waves_per_simd < 1 ? 1 : waves_per_simd] : 30.5;
}

constexpr int64_t kCUs = 256;
constexpr int64_t kLdsPerCU = 160 * 1024;
// waves per SIMD that the registers allow: the kernel that writes y uses <= 112 VGPRs,
// pass 1 <= 88 (512 per lane and SIMD)
constexpr int64_t kMaxWavesFull = 4, kMaxWavesLocal = 5;

// Relative time of one pass: `groups` workgroups of cg channels, `tiles` tiles each.
// A workgroup of more than 4 waves is counted as dealt to the CU's four SIMDs from the
// first, ceil(cg/32) on the busiest (as for the backward, where a second 6-wave
// workgroup was measured not to join the first; here, with CG = 48 on the 2.8B layer,
// 349 us against 249 us at CG = 80). The waves of workgroups of up to 4 waves spread
// over the SIMDs: k of them put ceil(k * waves / 4) on the busiest.
double pass_cost(int64_t groups, int64_t tiles, int cg, bool local) {
    const int64_t waves = cg / 8;
    const bool spread = waves <= 4;
    const int64_t per_simd = (waves + 3) / 4;
    const int64_t max_w = local ? kMaxWavesLocal : kMaxWavesFull;
    int64_t k = kLdsPerCU / scan_lds_bytes(cg, local);                  // by LDS
    const int64_t kw = spread ? max_w * 4 / waves : max_w / per_simd;    // by registers
    if (kw < k) k = kw;
    const int64_t per_cu = (groups + kCUs - 1) / kCUs;
    if (k > per_cu) k = per_cu;
    if (k < 1) k = 1;
    const int64_t rounds = (groups + kCUs * k - 1) / (kCUs * k);
    const int64_t w = spread ? (k * waves + 3) / 4 : k * per_simd;      // busiest SIMD
    // pass 1 skips the readout and the output stage; a workgroup's set-up costs about
    // one tile
    return (double)rounds * (double)(tiles + 1) * (double)w * wave_cost(w) * (local ? 0.85 : 1.0);
}

struct PlanChoice {
    int cg;
    int64_t nchunks, chunk_len;
    double cost;
    int64_t busy;  // CUs with a workgroup of the pass that writes y
};

// lower modelled time; on a tie, fewer chunks, then more busy CUs
bool better(const PlanChoice& a, const PlanChoice& b) {
    if (b.cg == 0) return true;
    if (a.cost < b.cost * (1 - 1e-9)) return true;
    if (a.cost > b.cost * (1 + 1e-9)) return false;
    if (a.nchunks != b.nchunks) return a.nchunks < b.nchunks;
    return a.busy > b.busy;
}

// Cost of (cg, chunk_len): single pass when chunk_len >= seqlen, else pass 1 over all
// chunks but one, the carry, and pass 2 over every chunk.
PlanChoice plan_cost(int64_t batch, int64_t seqlen, int64_t dim, int cg, int64_t chunk_len) {
    const int64_t groups = batch * ((dim + cg - 1) / cg);
    const int64_t tile = ssm::kTokenTile;
    if (chunk_len >= seqlen) {
        return PlanChoice{cg, 1, seqlen, pass_cost(groups, (seqlen + tile - 1) / tile, cg, false),
                          groups < kCUs ? groups : kCUs};
    }
    const int64_t k = (seqlen + chunk_len - 1) / chunk_len;
    const int64_t tiles = chunk_len / tile;
    // two more launches (pass 1 and the carry), each worth about 75 units (~3.5 us:
    // a 1 x 256 x 16 scan runs 25 us in one pass, 17 us in chunks of 32 tokens)
    const double c = pass_cost(groups * (k - 1), tiles, cg, true) +
                     pass_cost(groups * k, tiles, cg, false) + (double)k * 2.0 + 150.0;
    return PlanChoice{cg, k, chunk_len, c, groups * k < kCUs ? groups * k : kCUs};
}

// Plan for a shape. Shared by the workspace query and the call, so both agree.
ssm_status make_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                     ssm_dtype io_dtype, const ssm_scan_options* opts, ssm::ScanPlan* plan) {
    if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
        return fail(SSM_ERR_INVALID_ARGUMENT, "io_dtype %d is not SSM_F32 or SSM_BF16",
                    (int)io_dtype);
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0)
        return fail(SSM_ERR_INVALID_ARGUMENT,
                    "sizes must be >= 1 (batch=%lld seqlen=%lld dim=%lld dstate=%lld)",
                    (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate);
    if (dstate != ssm::kDState)
        return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld: only dstate=16 is supported",
                    (long long)dstate);
    const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
    int64_t io_bytes;
    if (!bytes4(batch, dim, seqlen, elem, &io_bytes))
        return fail(SSM_ERR_INVALID_ARGUMENT, "tensor size overflows");
    if (seqlen > (int64_t(1) << 40))
        return fail(SSM_ERR_INVALID_ARGUMENT, "seqlen too large");
    int32_t req_plan = 0, req_cg = 0;
    int64_t req_chunk = 0;
    if (opts) {
        req_cg = opts->group_channels;
        if (req_cg != 0 && !(req_cg >= 16 && req_cg <= 96 && req_cg % 16 == 0))
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "ssm_scan_options.group_channels=%d not in {0, 16, 32, 48, 64, 80, 96}",
                        (int)req_cg);
        if (opts->plan < 0 || opts->plan > 3)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.plan=%d not in {0,1,2,3}",
                        (int)opts->plan);
        if (opts->chunk_len < 0 || opts->chunk_len % ssm::kTokenTile != 0)
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "ssm_scan_options.chunk_len=%lld must be a multiple of %d",
                        (long long)opts->chunk_len, ssm::kTokenTile);
        if (opts->reverse != 0 && opts->reverse != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.reverse=%d not 0 or 1",
                        (int)opts->reverse);
        if (opts->accumulate != 0 && opts->accumulate != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.accumulate=%d not 0 or 1",
                        (int)opts->accumulate);
        if (opts->structured_a != 0 && opts->structured_a != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.structured_a=%d not 0 or 1",
                        (int)opts->structured_a);
        req_plan = opts->plan;
        req_chunk = opts->chunk_len;
    }
    if (batch * ((dim + 31) / 32) >= (int64_t(1) << 30))
        return fail(SSM_ERR_INVALID_ARGUMENT, "batch*dim too large");
    if (req_plan == 3) {
        // the wave-scan plan: B/C widened into the workspace in its staged layout (64 KB
        // per batch row and 512-token segment), then one launch over every row
        *plan = ssm::ScanPlan{};
        plan->wavescan = 1;
        plan->nchunks = 1;
        plan->chunk_len = seqlen;
        const int64_t nseg = (seqlen + ssm::kWaveSegTokens - 1) / ssm::kWaveSegTokens;
        int64_t bytes;
        if (!bytes4(batch, nseg, 2 * ssm::kDState * ssm::kWaveSegTokens, 4, &bytes))
            return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
        plan->ws_bcq = 0;
        plan->ws_total = align_up((size_t)bytes, 256);
        return SSM_OK;
    }
    const int64_t lpad = (seqlen + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;

    // Channels per workgroup and chunking: the choice with the lowest modelled time
    // (pass_cost above) among group sizes 16..96 and chunk counts 1 (single pass), 2,
    // 3, 4, 6, 8, 12, ... A requested group size, plan or chunk length restricts the
    // search. Ties go to fewer chunks, then to the candidate order: 16 channels first --
    // several 2-wave workgroups per CU run out of phase, their core at raised priority,
    // and none waits at a barrier for a busier SIMD (the 2.8B layer: 215 us at 16
    // against 241 us at 80, the 130M layer 160 against 163 us at 32, both ties in the
    // model) -- then larger groups, except that 32 channels come before 48: several
    // 4-wave workgroups per CU beat one 6-wave workgroup whose SIMDs hold 2, 2, 1, 1
    // waves (the 130M layer: 167 us at 32 against 181 us at 48, which the model ties).
    static const int kCands[] = {16, 96, 80, 64, 32, 48};
    PlanChoice best{0, 0, 0, 1e300, 0};
    for (int c : kCands) {
        if (req_cg && c != req_cg) continue;
        if (req_plan != 2) {
            const PlanChoice pc = plan_cost(batch, seqlen, dim, c, seqlen);
            if (better(pc, best)) best = pc;
        }
        if (req_plan == 1) continue;
        if (req_chunk > 0) {
            if (req_chunk < seqlen) {
                const PlanChoice pc = plan_cost(batch, seqlen, dim, c, req_chunk);
                if (better(pc, best)) best = pc;
            } else if (req_plan == 2 && best.cg == 0) {
                best = plan_cost(batch, seqlen, dim, c, seqlen);
            }
            continue;
        }
        for (int64_t kk = 2; kk <= 4096; kk = kk < 4 ? kk + 1 : kk + kk / 2) {
            int64_t cl = (seqlen + kk - 1) / kk;
            cl = (cl + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;
            if (cl >= seqlen) {
                if (req_plan == 2 && best.cg == 0) best = plan_cost(batch, seqlen, dim, c, seqlen);
                continue;
            }
            const PlanChoice pc = plan_cost(batch, seqlen, dim, c, cl);
            if (better(pc, best)) best = pc;
            if (cl <= ssm::kTokenTile) break;
        }
    }
    if (best.cg == 0) best = plan_cost(batch, seqlen, dim, req_cg ? req_cg : 32, seqlen);
    const int cg = best.cg;
    const int64_t ngroups = batch * ((dim + cg - 1) / cg);
    const int64_t nchunks = best.nchunks;
    const int64_t chunk_len = best.chunk_len;
    if (ngroups * nchunks >= (int64_t(1) << 31))
        return fail(SSM_ERR_INVALID_ARGUMENT, "too many chunks (%lld)", (long long)nchunks);
    int64_t bcq_bytes, st_bytes = 0, sum_bytes = 0, flag_bytes = 0;
    if (!bytes4(batch, lpad, 4 * 8, 4, &bcq_bytes))
        return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
    if (nchunks > 1) {
        if (!bytes4(batch * dim, nchunks, ssm::kDState, 4, &st_bytes) ||
            !bytes4(batch * dim, nchunks, 1, 4, &sum_bytes))
            return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
        flag_bytes = nchunks * 4;
    }
    plan->group_channels = cg;
    plan->ngroups = ngroups;
    plan->nchunks = (int)nchunks;
    plan->chunk_len = chunk_len;
    plan->ws_bcq = 0;
    plan->ws_state = align_up((size_t)bcq_bytes, 256);
    plan->ws_sum = align_up(plan->ws_state + (size_t)st_bytes, 256);
    plan->ws_flag = align_up(plan->ws_sum + (size_t)sum_bytes, 256);
    plan->ws_total = align_up(plan->ws_flag + (size_t)flag_bytes, 256);
    return SSM_OK;
}

constexpr int kBwdTile = 16;   // tokens per backward tile: a checkpoint every kBwdTile tokens
bool saved_layout(int64_t batch, int64_t seqlen, int64_t dim, ssm_dtype io_dtype, size_t* ws_q,
                  size_t* total);

ssm_status scan_impl(const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const void* z, const float* delta_bias,
                     int delta_softplus, const int32_t* cu_seqlens, int64_t nseq,
                     const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen,
                     int64_t dim, int64_t dstate, ssm_dtype io_dtype, void* workspace,
                     size_t workspace_bytes, const ssm_scan_options* opts, void* stream,
                     bool use_scratch = false) {
    const bool packed = cu_seqlens != nullptr;
    ssm::ScanPlan plan;
    ssm_status st = make_plan(batch, seqlen, dim, dstate, io_dtype, opts, &plan);
    if (st != SSM_OK) return st;
    // Packed sequences resumed in place (h_final == h0): in the chunked plan the workgroup
    // of a sequence's last chunk writes its final state while the workgroup of its first
    // chunk, in the same launch, may still read its initial state. The single pass reads
    // a sequence's h0 before it writes its h_final, in the same thread; its workspace is
    // no larger than the chunked plan's, so the caller's buffer still fits.
    if (packed && h_final && (const void*)h_final == (const void*)h0 && plan.nchunks > 1) {
        if (opts && opts->plan == 2)
            return fail(SSM_ERR_UNSUPPORTED,
                        "packed sequences with h_final == h0 (in place) run in the single-pass "
                        "plan only; ssm_scan_options.plan = 2 asks for the chunked plan");
        ssm_scan_options one = opts ? *opts : ssm_scan_options{};
        one.plan = 1;
        one.chunk_len = 0;
        st = make_plan(batch, seqlen, dim, dstate, io_dtype, &one, &plan);
        if (st != SSM_OK) return st;
    }
    if (delta_softplus != 0 && delta_softplus != 1)
        return fail(SSM_ERR_INVALID_ARGUMENT, "delta_softplus must be 0 or 1");
    if (!x || !delta || !A || !B || !C || !y)
        return fail(SSM_ERR_INVALID_ARGUMENT,
                    "x, delta, A, B, C and y are required (got x=%p delta=%p A=%p B=%p "
                    "C=%p y=%p)",
                    x, delta, (const void*)A, B, C, y);
    const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
    const int64_t io = batch * dim * seqlen * elem;
    const int64_t bc = batch * seqlen * dstate * elem;
    // per-row states: one per batch row, or one per packed sequence
    const int64_t nstates = packed ? nseq : batch;
    int64_t st_b;
    if (!bytes4(nstates, dim, dstate, 4, &st_b))
        return fail(SSM_ERR_INVALID_ARGUMENT, "state size overflows");
    struct {
        const char* name;
        const void* p;
        uintptr_t align;
    } al[] = {{"x", x, 16},       {"delta", delta, 16}, {"z", z, 16},
              {"y", y, 16},       {"B", B, 16},         {"C", C, 16},
              {"h0", h0, 16},     {"h_final", h_final, 16},
              {"A", A, 16},       {"D", D, 4},          {"delta_bias", delta_bias, 4},
              {"cu_seqlens", cu_seqlens, 4},            {"workspace", workspace, 16}};
    for (auto& a : al)
        if (a.p && !aligned(a.p, a.align))
            return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                        (unsigned)a.align);
    // use_scratch (ssm_scan_fwd_noalloc): the workspace is the library's static scratch,
    // looked up after every check below; it overlaps no caller buffer
    if (use_scratch && plan.ws_total > ssm::kScratchBytes)
        return fail(SSM_ERR_UNSUPPORTED,
                    "this shape and plan need %zu bytes of workspace; the static scratch of "
                    "ssm_scan_fwd_noalloc holds %zu (call ssm_scan_fwd with a workspace)",
                    plan.ws_total, ssm::kScratchBytes);
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
    } else if (plan.ws_total > 0 && (!workspace || workspace_bytes < plan.ws_total)) {
        return fail(SSM_ERR_WORKSPACE_TOO_SMALL,
                    "workspace needs %zu bytes (got %zu at %p)", plan.ws_total,
                    workspace_bytes, workspace);
    }
    const Region ry = region("y", y, io);
    const Region rhf = region("h_final", h_final, st_b);
    const Region rws = region("workspace", workspace, (int64_t)plan.ws_total);
    const Region inputs[] = {region("x", x, io),
                             region("delta", delta, io),
                             region("z", z, io),
                             region("B", B, bc),
                             region("C", C, bc),
                             region("A", A, dim * dstate * 4),
                             region("D", D, dim * 4),
                             region("delta_bias", delta_bias, dim * 4),
                             region("cu_seqlens", cu_seqlens, (nseq + 1) * 4),
                             region("h0", h0, st_b)};
    const Region& rh0 = inputs[9];
    for (const Region& r : inputs) {
        if (overlaps(ry, r))
            return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps %s", r.name);
        if (overlaps(rws, r))
            return fail(SSM_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
        if (h_final && overlaps(rhf, r)) {
            const bool same_h0 = (&r == &rh0) && (const void*)h_final == h0;
            if (!same_h0)
                return fail(SSM_ERR_INVALID_ARGUMENT,
                            "h_final overlaps %s (only h_final == h0 exactly is allowed)",
                            r.name);
        }
    }
    if (h_final && overlaps(ry, rhf))
        return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps h_final");
    if (overlaps(rws, ry)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace overlaps y");
    if (h_final && overlaps(rws, rhf))
        return fail(SSM_ERR_INVALID_ARGUMENT, "workspace overlaps h_final");

    if (plan.wavescan && (packed || (opts && opts->save_workspace)))
        return fail(SSM_ERR_UNSUPPORTED,
                    "ssm_scan_options.plan = 3 (wave scan) takes batch rows without "
                    "save_workspace");
    // training: also save the checkpoints and q for the backward
    void* const save = opts ? opts->save_workspace : nullptr;
    if (opts && opts->saved)
        return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.saved is an option of ssm_scan_bwd");
    size_t save_q = 0, save_total = 0;
    if (save) {
        if (packed || opts->accumulate)
            return fail(SSM_ERR_UNSUPPORTED,
                        "save_workspace: scans of ssm_scan_fwd (batch rows) without accumulate "
                        "only");
        if (!saved_layout(batch, seqlen, dim, io_dtype, &save_q, &save_total))
            return fail(SSM_ERR_INVALID_ARGUMENT, "save_workspace size overflows");
        if (!aligned(save, 16))
            return fail(SSM_ERR_UNSUPPORTED, "save_workspace=%p is not 16-byte aligned", save);
        if (opts->save_workspace_bytes < save_total)
            return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "save_workspace needs %zu bytes (got %zu)",
                        save_total, opts->save_workspace_bytes);
        const Region rsv = region("save_workspace", save, (int64_t)save_total);
        for (const Region& r : inputs)
            if (overlaps(rsv, r))
                return fail(SSM_ERR_INVALID_ARGUMENT, "save_workspace overlaps %s", r.name);
        if (overlaps(rsv, ry) || (h_final && overlaps(rsv, rhf)) || overlaps(rsv, rws))
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "save_workspace overlaps y, h_final or the workspace");
    }

    if (use_scratch) {
        const hipError_t e = ssm::scratch_address(static_cast<hipStream_t>(stream), &workspace);
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    }
    ssm::ScanParams prm{};
    char* ws = static_cast<char*>(workspace);
    prm.x = x;
    prm.delta = delta;
    prm.z = z;
    prm.y = y;
    prm.A = A;
    prm.D = D;
    prm.bias = delta_bias;
    prm.h0 = h0;
    prm.h_final = h_final;
    prm.bcq = reinterpret_cast<float*>(ws + plan.ws_bcq);
    prm.chunk_state = plan.nchunks > 1 ? reinterpret_cast<float*>(ws + plan.ws_state) : nullptr;
    prm.chunk_sum = plan.nchunks > 1 ? reinterpret_cast<float*>(ws + plan.ws_sum) : nullptr;
    prm.chunk_flag = plan.nchunks > 1 ? reinterpret_cast<int32_t*>(ws + plan.ws_flag) : nullptr;
    prm.cu = cu_seqlens;
    prm.nseq = (int32_t)nseq;
    prm.batch = batch;
    prm.seqlen = seqlen;
    prm.dim = dim;
    prm.lpad = (seqlen + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;
    prm.chunk_len = plan.chunk_len;
    prm.nchunks = plan.nchunks;
    prm.groups_per_batch = (int32_t)((dim + plan.group_channels - 1) / plan.group_channels);
    prm.ngroups = (int32_t)(batch * prm.groups_per_batch);
    prm.chunk_offset = 0;
    prm.softplus = delta_softplus;
    prm.aligned = ((seqlen * elem) % 16) == 0;
    prm.reverse = opts ? opts->reverse : 0;
    prm.accumulate = opts ? opts->accumulate : 0;
    prm.structured_a = opts ? opts->structured_a : 0;
    if (save) {
        prm.ckpt = static_cast<float*>(save);
        prm.nckpt = (seqlen + kBwdTile - 1) / kBwdTile;
        prm.q = static_cast<char*>(save) + save_q;
    }
    if (getenv("SSMSCAN_LOG"))
        fprintf(stderr,
                "[ssmscan] scan b=%lld L=%lld d=%lld %s%s%s%s: %s, %d channels/group, %lld "
                "groups, chunks=%d x %lld\n",
                (long long)batch, (long long)seqlen, (long long)dim,
                io_dtype == SSM_BF16 ? "bf16" : "f32", packed ? " packed" : "",
                prm.reverse ? " reverse" : "", prm.accumulate ? " accumulate" : "",
                plan.wavescan ? "wave scan" : plan.nchunks > 1 ? "chunked" : "single pass",
                plan.group_channels,
                (long long)plan.ngroups, plan.nchunks, (long long)plan.chunk_len);
    hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->timing_begin) : nullptr;
    hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->timing_end) : nullptr;
    const hipError_t e =
        plan.wavescan ? ssm::launch_wavescan(prm, B, C, io_dtype == SSM_BF16,
                                             static_cast<hipStream_t>(stream), ev0, ev1)
                      : ssm::launch_scan(plan, prm, B, C, io_dtype == SSM_BF16,
                                         static_cast<hipStream_t>(stream), ev0, ev1);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return SSM_OK;
}

// ---- backward ---------------------------------------------------------------------

// LDS bytes of one backward workgroup of cg channels (must match scan_bwd_kernel):
// Delta, u, dq [cg][20]; two [8][cg][16] partial arrays; two B/C tiles of 8 x (16 x 4 + 4)
// floats; row sums [16][cg/2][4].
int64_t bwd_lds_bytes(int cg) { return (int64_t)(348 * cg + 1088) * 4; }

// Relative time of one backward pass: `groups` workgroups of cg channels over `tiles`
// 16-token tiles (as pass_cost, with the backward's LDS and its <= 168 VGPRs: 3 waves
// per SIMD). A workgroup's cg/8 waves are counted as dealt to the CU's four SIMDs from
// the first one, so it puts ceil(cg/32) of them on its busiest SIMD, and a second
// 6-wave workgroup (cg = 48) does not fit beside the first: measured on the 2.8B layer,
// the backward kernel takes 1039 us with 48 channels per workgroup, 773 us with 64 (one
// 8-wave workgroup per CU) and 728 us with 32 (three 4-wave workgroups per CU); on the
// 130M layer 536, 458 and 380 us.
double bwd_pass_cost(int64_t groups, int64_t tiles, int cg) {
    const int64_t per_simd = (cg / 8 + 3) / 4;
    int64_t k = kLdsPerCU / bwd_lds_bytes(cg);
    const int64_t kw = 3 / per_simd;
    if (kw < k) k = kw;
    const int64_t per_cu = (groups + kCUs - 1) / kCUs;
    if (k > per_cu) k = per_cu;
    if (k < 1) k = 1;
    const int64_t rounds = (groups + kCUs * k - 1) / (kCUs * k);
    const int64_t w = k * per_simd;
    return (double)rounds * (double)(tiles + 1) * (double)w * wave_cost(w);
}

struct BwdPlan {
    ssm::ScanPlan fwd;      // the forward pass that writes q and the checkpoints
    int cg;
    int64_t nckpt, chunk_len, nchunks;
    // workspace offsets: the checkpoints and q first (what a training forward saves;
    // their place depends on the shape only), then the forward's own workspace
    size_t ws_ckpt, ws_q, ws_fwd, ws_bc, ws_A, ws_D, ws_bias, ws_gc, ws_gs, ws_flag, ws_ev,
        ws_seq, ws_total;
};

// Where the checkpoints ([batch][ceil(L/16)][dim][16] fp32, offset 0) and q ([batch][dim][L]
// io) start a backward workspace, and the bytes they take. False on overflow.
bool saved_layout(int64_t batch, int64_t seqlen, int64_t dim, ssm_dtype io_dtype, size_t* ws_q,
                  size_t* total) {
    const int64_t nckpt = (seqlen + kBwdTile - 1) / kBwdTile;
    const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
    int64_t ck, qb;
    if (!bytes4(batch * dim, nckpt, ssm::kDState, 4, &ck) ||
        !bytes4(batch * dim, seqlen, elem, 1, &qb))
        return false;
    *ws_q = align_up((size_t)ck, 256);
    *total = *ws_q + (size_t)qb;
    return true;
}

// Channels per backward workgroup and chunking of the sequence (the cost model of
// make_plan: pass 1 of the chunked backward -- only the gradient chain -- costs about a
// quarter of a full pass).
// The backward kernel addresses a workgroup's cg rows of [batch][dim][L] with 32-bit
// byte offsets: cg * L * elem must stay below 2^32.
bool bwd_rows_fit(int cg, int64_t seqlen, int64_t elem) {
    return (int64_t)cg * seqlen * elem < (int64_t(1) << 32);
}

// Returns false when no allowed channel group fits (the sequence is too long).
bool choose_bwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t elem, int req_cg,
                     int64_t req_chunk, BwdPlan* bp) {
    static const int kCands[] = {64, 48, 32};
    const int64_t tile = 16;
    double best_c = 1e300;
    bp->cg = 0;
    bp->chunk_len = seqlen;
    bp->nchunks = 1;
    for (int cg : kCands) {
        if (req_cg && cg != req_cg) continue;
        if (!bwd_rows_fit(cg, seqlen, elem)) continue;
        const int64_t groups = batch * ((dim + cg - 1) / cg);
        for (int64_t kk = 1; kk <= 4096; kk = kk < 4 ? kk + 1 : kk + kk / 2) {
            int64_t cl = seqlen;
            if (req_chunk > 0) {
                cl = req_chunk;
            } else if (kk > 1) {
                cl = (seqlen + kk - 1) / kk;
                cl = (cl + 31) / 32 * 32;
            }
            const int64_t k = (seqlen + cl - 1) / cl;
            if (req_chunk == 0 && kk > 1 && (cl >= seqlen || cl < 256)) break;
            const int64_t tiles = (cl + tile - 1) / tile;
            double c = bwd_pass_cost(groups * k, tiles, cg);
            if (k > 1) c += 0.25 * bwd_pass_cost(groups * (k - 1), tiles, cg) + 300.0;
            if (c < best_c * (1 - 1e-9)) {
                best_c = c;
                bp->cg = cg;
                bp->chunk_len = k > 1 ? cl : seqlen;
                bp->nchunks = k;
            }
            if (req_chunk > 0) break;
        }
    }
    return bp->cg != 0;
}

ssm_status make_bwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         ssm_dtype io_dtype, const ssm_scan_options* opts, BwdPlan* bp) {
    if (opts && opts->accumulate)
        return fail(SSM_ERR_UNSUPPORTED, "the backward scan takes no accumulate option");
    if (opts && opts->plan == 3)
        return fail(SSM_ERR_UNSUPPORTED,
                    "the backward's checkpoint pass runs plan 1 or 2, not the wave scan (3)");
    if (opts && opts->save_workspace)
        return fail(SSM_ERR_INVALID_ARGUMENT,
                    "ssm_scan_options.save_workspace is an option of ssm_scan_fwd");
    if (opts && opts->saved != 0 && opts->saved != 1)
        return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.saved=%d must be 0 or 1",
                    opts->saved);
    ssm_status st = make_plan(batch, seqlen, dim, dstate, io_dtype, opts, &bp->fwd);
    if (st != SSM_OK) return st;
    const int req = opts ? opts->bwd_group_channels : 0;
    if (req != 0 && req != 32 && req != 48 && req != 64)
        return fail(SSM_ERR_INVALID_ARGUMENT,
                    "ssm_scan_options.bwd_group_channels=%d not in {0, 32, 48, 64}", req);
    const int64_t req_chunk = opts ? opts->bwd_chunk_len : 0;
    if (req_chunk < 0 || req_chunk % 32 != 0)
        return fail(SSM_ERR_INVALID_ARGUMENT,
                    "ssm_scan_options.bwd_chunk_len=%lld must be a multiple of 32",
                    (long long)req_chunk);
    const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
    if (!choose_bwd_plan(batch, seqlen, dim, elem, req, req_chunk, bp))
        return fail(SSM_ERR_UNSUPPORTED,
                    "ssm_scan_bwd: seqlen=%lld is too long for one row (a workgroup's rows must "
                    "span less than 4 GiB: seqlen < %lld for this dtype%s)",
                    (long long)seqlen, (long long)(((int64_t)1 << 32) / ((req ? req : 32) * elem)),
                    req ? " and bwd_group_channels" : "");
    const int64_t gpb = (dim + bp->cg - 1) / bp->cg;
    const int64_t K = bp->nchunks;
    bp->nckpt = (seqlen + kBwdTile - 1) / kBwdTile;
    int64_t ck, qb, bc, pa, pd, gc = 0, gs = 0;
    if (!bytes4(batch * dim, bp->nckpt, ssm::kDState, 4, &ck) ||
        !bytes4(batch * dim, seqlen, elem, 1, &qb) || !bytes4(batch * gpb, seqlen, 32, 4, &bc) ||
        !bytes4(batch * K, dim, ssm::kDState, 4, &pa) || !bytes4(batch * K, dim, 1, 4, &pd) ||
        (K > 1 && (!bytes4(batch * dim, K, ssm::kDState, 4, &gc) ||
                   !bytes4(batch * dim, K, 1, 4, &gs))))
        return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
    if (batch * gpb * K >= (int64_t(1) << 31))
        return fail(SSM_ERR_INVALID_ARGUMENT, "too many backward chunks");
    size_t saved_total = 0;
    if (!saved_layout(batch, seqlen, dim, io_dtype, &bp->ws_q, &saved_total))
        return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
    bp->ws_ckpt = 0;
    bp->ws_fwd = align_up(saved_total, 256);
    bp->ws_bc = align_up(bp->ws_fwd + bp->fwd.ws_total, 256);
    bp->ws_A = align_up(bp->ws_bc + (size_t)bc, 256);
    bp->ws_D = align_up(bp->ws_A + (size_t)pa, 256);
    bp->ws_bias = align_up(bp->ws_D + (size_t)pd, 256);
    bp->ws_gc = align_up(bp->ws_bias + (size_t)pd, 256);
    bp->ws_gs = align_up(bp->ws_gc + (size_t)gc, 256);
    bp->ws_flag = align_up(bp->ws_gs + (size_t)gs, 256);   // [K] int32 (packed input)
    bp->ws_ev = align_up(bp->ws_flag + (size_t)K * 4, 256);  // [ceil(L/16)] u32 (packed)
    bp->ws_seq = align_up(bp->ws_ev + (size_t)bp->nckpt * 4, 256);   // [L] int32 (packed)
    bp->ws_total = align_up(bp->ws_seq + (size_t)seqlen * 4, 256);
    return SSM_OK;
}

// The backward of ssm_scan_bwd (cu == nullptr: batch rows) and of ssm_scan_varlen_bwd
// (cu set: batch = 1, seqlen = total, h0 / dh_final / dh0 per sequence).
ssm_status bwd_impl(const void* x, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int delta_softplus, const float* h0, const int32_t* cu, int64_t nseq,
                    const void* dy, const float* dh_final, void* dx, void* ddelta, void* dz,
                    float* dA, float* dB, float* dC, float* dD, float* ddelta_bias, float* dh0,
                    int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    ssm_dtype io_dtype, void* workspace, size_t workspace_bytes,
                    const ssm_scan_options* opts, void* stream) {
    try {
        BwdPlan bp;
        ssm_status st = make_bwd_plan(batch, seqlen, dim, dstate, io_dtype, opts, &bp);
        if (st != SSM_OK) return st;
        if (delta_softplus != 0 && delta_softplus != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "delta_softplus must be 0 or 1");
        if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC)
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "x, delta, A, B, C, dy, dx, ddelta, dA, dB and dC are required");
        if ((z != nullptr) != (dz != nullptr))
            return fail(SSM_ERR_INVALID_ARGUMENT, "dz is required exactly when z is given");
        if (dD && !D) return fail(SSM_ERR_INVALID_ARGUMENT, "dD needs D");
        if (ddelta_bias && !delta_bias)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ddelta_bias needs delta_bias");
        const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
        const int64_t io = batch * dim * seqlen * elem;
        const int64_t bc = batch * seqlen * dstate * elem;
        const int64_t bc32 = batch * seqlen * dstate * 4;
        const int64_t nstates = cu ? nseq : batch;   // rows of h0, dh_final, dh0
        int64_t stb;
        if (!bytes4(nstates, dim, dstate, 4, &stb))
            return fail(SSM_ERR_INVALID_ARGUMENT, "state size overflows");
        if (cu && opts && opts->saved)
            return fail(SSM_ERR_UNSUPPORTED,
                        "ssm_scan_varlen_bwd recomputes its checkpoints (saved must be 0)");
        const int32_t reverse = opts ? opts->reverse : 0;
        struct {
            const char* name;
            const void* p;
            uintptr_t align;
        } al[] = {{"x", x, 16},           {"delta", delta, 16}, {"z", z, 16},
                  {"dy", dy, 16},         {"B", B, 16},         {"C", C, 16},
                  {"A", A, 16},           {"D", D, 4},          {"delta_bias", delta_bias, 4},
                  {"h0", h0, 16},         {"dh_final", dh_final, 16},
                  {"dx", dx, 16},         {"ddelta", ddelta, 16}, {"dz", dz, 16},
                  {"dA", dA, 16},         {"dB", dB, 16},       {"dC", dC, 16},
                  {"dD", dD, 4},          {"ddelta_bias", ddelta_bias, 4},
                  {"dh0", dh0, 16},       {"workspace", workspace, 16},
                  {"cu_seqlens", cu, 4}};
        for (auto& a : al)
            if (a.p && !aligned(a.p, a.align))
                return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                            (unsigned)a.align);
        if (!workspace || workspace_bytes < bp.ws_total)
            return fail(SSM_ERR_WORKSPACE_TOO_SMALL,
                        "workspace needs %zu bytes (got %zu at %p)", bp.ws_total,
                        workspace_bytes, workspace);
        const Region regs[] = {
            region("x", x, io),           region("delta", delta, io),
            region("z", z, io),           region("dy", dy, io),
            region("B", B, bc),           region("C", C, bc),
            region("A", A, dim * dstate * 4), region("D", D, dim * 4),
            region("delta_bias", delta_bias, dim * 4), region("h0", h0, stb),
            region("dh_final", dh_final, stb), region("cu_seqlens", cu, (nseq + 1) * 4),
            // outputs from here on: each may overlap nothing
            region("dx", dx, io),         region("ddelta", ddelta, io),
            region("dz", dz, io),         region("dA", dA, dim * dstate * 4),
            region("dB", dB, bc32),       region("dC", dC, bc32),
            region("dD", dD, dim * 4),    region("ddelta_bias", ddelta_bias, dim * 4),
            region("dh0", dh0, stb),      region("workspace", workspace, (int64_t)bp.ws_total)};
        constexpr int kFirstOut = 12;
        constexpr int kN = sizeof(regs) / sizeof(regs[0]);
        for (int i = kFirstOut; i < kN; ++i)
            for (int j = 0; j < kN; ++j)
                if (i != j && overlaps(regs[i], regs[j]))
                    return fail(SSM_ERR_INVALID_ARGUMENT, "%s overlaps %s", regs[i].name,
                                regs[j].name);

        char* ws = static_cast<char*>(workspace);
        char* fws = ws + bp.ws_fwd;   // the forward's own workspace
        hipStream_t strm = static_cast<hipStream_t>(stream);
        const bool saved = opts && opts->saved;
        // 1. B/C widening and the forward in checkpoint mode, with the forward's own
        //    plan: it writes q (the output before the gate: no z) and the state before
        //    every 16th token -- or, when the training forward saved those, the widening
        //    alone
        ssm::ScanParams fp{};
        fp.x = x;
        fp.delta = delta;
        fp.z = nullptr;
        fp.y = ws + bp.ws_q;
        fp.A = A;
        fp.D = D;
        fp.bias = delta_bias;
        fp.h0 = h0;
        fp.h_final = nullptr;
        fp.bcq = reinterpret_cast<float*>(fws + bp.fwd.ws_bcq);
        fp.chunk_state =
            bp.fwd.nchunks > 1 ? reinterpret_cast<float*>(fws + bp.fwd.ws_state) : nullptr;
        fp.chunk_sum =
            bp.fwd.nchunks > 1 ? reinterpret_cast<float*>(fws + bp.fwd.ws_sum) : nullptr;
        fp.chunk_flag =
            bp.fwd.nchunks > 1 ? reinterpret_cast<int32_t*>(fws + bp.fwd.ws_flag) : nullptr;
        fp.cu = cu;
        fp.nseq = (int32_t)nseq;
        fp.reverse = reverse;
        fp.ckpt = reinterpret_cast<float*>(ws + bp.ws_ckpt);
        fp.nckpt = bp.nckpt;
        fp.batch = batch;
        fp.seqlen = seqlen;
        fp.dim = dim;
        fp.lpad = (seqlen + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;
        fp.chunk_len = bp.fwd.chunk_len;
        fp.nchunks = bp.fwd.nchunks;
        fp.groups_per_batch =
            (int32_t)((dim + bp.fwd.group_channels - 1) / bp.fwd.group_channels);
        fp.ngroups = (int32_t)(batch * fp.groups_per_batch);
        fp.softplus = delta_softplus;
        fp.aligned = ((seqlen * elem) % 16) == 0;
        hipError_t e = saved ? ssm::launch_bc_widen(B, C, fp.bcq, batch, seqlen, fp.lpad,
                                                    io_dtype == SSM_BF16, strm)
                             : ssm::launch_scan(bp.fwd, fp, B, C, io_dtype == SSM_BF16, strm,
                                                nullptr, nullptr);
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        // 2. the backward kernel and its reductions
        ssm::BwdParams prm{};
        prm.x = x;
        prm.delta = delta;
        prm.z = z;
        prm.dy = dy;
        prm.A = A;
        prm.D = D;
        prm.bias = delta_bias;
        prm.dh_final = dh_final;
        prm.ckpt = fp.ckpt;
        prm.q = ws + bp.ws_q;
        prm.bcq = fp.bcq;
        prm.dx = dx;
        prm.ddelta = ddelta;
        prm.dz = dz;
        prm.dA = dA;
        prm.dB = dB;
        prm.dC = dC;
        prm.dD = dD;
        prm.dbias = ddelta_bias;
        prm.dh0 = dh0;
        prm.part_bc = reinterpret_cast<float*>(ws + bp.ws_bc);
        prm.part_A = reinterpret_cast<float*>(ws + bp.ws_A);
        prm.part_D = reinterpret_cast<float*>(ws + bp.ws_D);
        prm.part_bias = reinterpret_cast<float*>(ws + bp.ws_bias);
        prm.g_carry = bp.nchunks > 1 ? reinterpret_cast<float*>(ws + bp.ws_gc) : nullptr;
        prm.g_sum = bp.nchunks > 1 ? reinterpret_cast<float*>(ws + bp.ws_gs) : nullptr;
        prm.cu = cu;
        prm.nseq = (int32_t)nseq;
        prm.h0 = h0;
        prm.chunk_flag = reinterpret_cast<int32_t*>(ws + bp.ws_flag);
        prm.reverse = reverse;
        prm.tile_ev = reinterpret_cast<uint32_t*>(ws + bp.ws_ev);
        prm.tok_seq = reinterpret_cast<int32_t*>(ws + bp.ws_seq);
        prm.chunk_len = bp.chunk_len;
        prm.nchunks = (int32_t)bp.nchunks;
        prm.chunk_offset = 0;
        prm.batch = batch;
        prm.seqlen = seqlen;
        prm.dim = dim;
        prm.lpad = fp.lpad;
        prm.nckpt = bp.nckpt;
        prm.groups_per_batch = (int32_t)((dim + bp.cg - 1) / bp.cg);
        prm.softplus = delta_softplus;
        prm.aligned = fp.aligned;
        if (getenv("SSMSCAN_LOG"))
            fprintf(stderr,
                    "[ssmscan] bwd b=%lld L=%lld d=%lld %s: checkpoint pass %s%d channels/group "
                    "x %d chunks, backward %d channels/group x %lld chunks of %lld\n",
                    (long long)batch, (long long)seqlen, (long long)dim,
                    io_dtype == SSM_BF16 ? "bf16" : "f32", saved ? "(saved by the forward) " : "",
                    bp.fwd.group_channels, bp.fwd.nchunks, bp.cg, (long long)bp.nchunks,
                    (long long)bp.chunk_len);
        hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->timing_begin) : nullptr;
        hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->timing_end) : nullptr;
        e = ssm::launch_scan_bwd(bp.cg, prm, io_dtype == SSM_BF16, strm, ev0, ev1);
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return SSM_OK;
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

}  // namespace

extern "C" {

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    ssm_dtype io_dtype, const ssm_scan_options* opts) {
    BwdPlan bp;
    if (make_bwd_plan(batch, seqlen, dim, dstate, io_dtype, opts, &bp) != SSM_OK) return 0;
    return bp.ws_total;
}

ssm_status ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z,
                        const float* delta_bias, int delta_softplus, const float* h0,
                        const void* dy, const float* dh_final, void* dx, void* ddelta,
                        void* dz, float* dA, float* dB, float* dC, float* dD,
                        float* ddelta_bias, float* dh0, int64_t batch, int64_t seqlen,
                        int64_t dim, int64_t dstate, ssm_dtype io_dtype, void* workspace,
                        size_t workspace_bytes, const ssm_scan_options* opts, void* stream) {
    return bwd_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, nullptr, 0, dy,
                    dh_final, dx, ddelta, dz, dA, dB, dC, dD, ddelta_bias, dh0, batch, seqlen,
                    dim, dstate, io_dtype, workspace, workspace_bytes, opts, stream);
}

size_t ssm_scan_varlen_bwd_workspace_bytes(int64_t total, int64_t dim, int64_t dstate,
                                           ssm_dtype io_dtype, const ssm_scan_options* opts) {
    if (total == 0) return 0;
    return ssm_scan_bwd_workspace_bytes(1, total, dim, dstate, io_dtype, opts);
}

ssm_status ssm_scan_varlen_bwd(const void* x, const void* delta, const float* A, const void* B,
                               const void* C, const float* D, const void* z,
                               const float* delta_bias, int delta_softplus,
                               const int32_t* cu_seqlens, int64_t nseq, const float* h0,
                               const void* dy, const float* dh_final, void* dx, void* ddelta,
                               void* dz, float* dA, float* dB, float* dC, float* dD,
                               float* ddelta_bias, float* dh0, int64_t total, int64_t dim,
                               int64_t dstate, ssm_dtype io_dtype, void* workspace,
                               size_t workspace_bytes, const ssm_scan_options* opts,
                               void* stream) {
    try {
        if (!cu_seqlens) return fail(SSM_ERR_INVALID_ARGUMENT, "cu_seqlens is required");
        if (nseq < 1 || nseq >= (int64_t(1) << 30))
            return fail(SSM_ERR_INVALID_ARGUMENT, "nseq=%lld must be in [1, 2^30)",
                        (long long)nseq);
        if (total < 0 || total >= (int64_t(1) << 31))
            return fail(SSM_ERR_INVALID_ARGUMENT, "total=%lld must be in [0, 2^31)",
                        (long long)total);
        if (total > 0)
            return bwd_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, cu_seqlens,
                            nseq, dy, dh_final, dx, ddelta, dz, dA, dB, dC, dD, ddelta_bias,
                            dh0, 1, total, dim, dstate, io_dtype, workspace, workspace_bytes,
                            opts, stream);
        // no tokens: every sequence is empty (dh0 = dh_final) and the sums over tokens are 0
        BwdPlan bp;
        ssm_status st = make_bwd_plan(1, 1, dim, dstate, io_dtype, opts, &bp);
        if (st != SSM_OK) return st;
        if (delta_softplus != 0 && delta_softplus != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "delta_softplus must be 0 or 1");
        if (!dA) return fail(SSM_ERR_INVALID_ARGUMENT, "dA is required");
        if (dD && !D) return fail(SSM_ERR_INVALID_ARGUMENT, "dD needs D");
        if (ddelta_bias && !delta_bias)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ddelta_bias needs delta_bias");
        int64_t stb;
        if (!bytes4(nseq, dim, dstate, 4, &stb))
            return fail(SSM_ERR_INVALID_ARGUMENT, "state size overflows");
        struct {
            const char* name;
            const void* p;
            uintptr_t align;
        } al[] = {{"dA", dA, 16}, {"dD", dD, 4}, {"ddelta_bias", ddelta_bias, 4},
                  {"dh0", dh0, 16}, {"dh_final", dh_final, 16}};
        for (auto& a : al)
            if (a.p && !aligned(a.p, a.align))
                return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                            (unsigned)a.align);
        const Region regs[] = {region("dh_final", dh_final, stb), region("dA", dA, dim * dstate * 4),
                               region("dD", dD, dim * 4), region("ddelta_bias", ddelta_bias, dim * 4),
                               region("dh0", dh0, stb)};
        for (int i = 1; i < 5; ++i)
            for (int j = 0; j < 5; ++j)
                if (i != j && overlaps(regs[i], regs[j]))
                    return fail(SSM_ERR_INVALID_ARGUMENT, "%s overlaps %s", regs[i].name,
                                regs[j].name);
        hipStream_t strm = static_cast<hipStream_t>(stream);
        hipError_t e = ssm::launch_copy_state(nullptr, dA, dim * dstate, strm);
        if (e == hipSuccess && dD) e = ssm::launch_copy_state(nullptr, dD, dim, strm);
        if (e == hipSuccess && ddelta_bias)
            e = ssm::launch_copy_state(nullptr, ddelta_bias, dim, strm);
        if (e == hipSuccess && dh0) e = ssm::launch_copy_state(dh_final, dh0, stb / 4, strm);
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return SSM_OK;
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}


const char* ssm_status_string(ssm_status s) {
    switch (s) {
        case SSM_OK: return "ok";
        case SSM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SSM_ERR_UNSUPPORTED: return "unsupported";
        case SSM_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SSM_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* ssm_last_error(void) { return g_last_error; }

int ssm_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                ssm_dtype io_dtype, const ssm_scan_options* opts) {
    ssm::ScanPlan plan;
    if (make_plan(batch, seqlen, dim, dstate, io_dtype, opts, &plan) != SSM_OK) return 0;
    return plan.ws_total;
}

ssm_status ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z,
                        const float* delta_bias, int delta_softplus, const float* h0,
                        void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t dim,
                        int64_t dstate, ssm_dtype io_dtype, void* workspace,
                        size_t workspace_bytes, const ssm_scan_options* opts, void* stream) {
    try {
        return scan_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, nullptr, 0, h0, y,
                         h_final, batch, seqlen, dim, dstate, io_dtype, workspace,
                         workspace_bytes, opts, stream);
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

ssm_status ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B,
                                const void* C, const float* D, const void* z,
                                const float* delta_bias, int delta_softplus, const float* h0,
                                void* y, float* h_final, int64_t batch, int64_t seqlen,
                                int64_t dim, int64_t dstate, ssm_dtype io_dtype,
                                const ssm_scan_options* opts, void* stream) {
    try {
        return scan_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, nullptr, 0, h0, y,
                         h_final, batch, seqlen, dim, dstate, io_dtype, nullptr, 0, opts, stream,
                         /*use_scratch=*/true);
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

size_t ssm_scan_varlen_workspace_bytes(int64_t total, int64_t dim, int64_t dstate,
                                       ssm_dtype io_dtype, const ssm_scan_options* opts) {
    if (total == 0) return 0;
    return ssm_scan_workspace_bytes(1, total, dim, dstate, io_dtype, opts);
}

ssm_status ssm_scan_varlen_fwd(const void* x, const void* delta, const float* A, const void* B,
                               const void* C, const float* D, const void* z,
                               const float* delta_bias, int delta_softplus,
                               const int32_t* cu_seqlens, int64_t nseq, const float* h0,
                               void* y, float* h_final, int64_t total, int64_t dim,
                               int64_t dstate, ssm_dtype io_dtype, void* workspace,
                               size_t workspace_bytes, const ssm_scan_options* opts,
                               void* stream) {
    try {
        if (!cu_seqlens)
            return fail(SSM_ERR_INVALID_ARGUMENT, "cu_seqlens is required");
        if (nseq < 1 || nseq >= (int64_t(1) << 30))
            return fail(SSM_ERR_INVALID_ARGUMENT, "nseq=%lld must be in [1, 2^30)",
                        (long long)nseq);
        if (total < 0 || total >= (int64_t(1) << 31))
            return fail(SSM_ERR_INVALID_ARGUMENT, "total=%lld must be in [0, 2^31)",
                        (long long)total);
        if (total > 0)
            return scan_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, cu_seqlens,
                             nseq, h0, y, h_final, 1, total, dim, dstate, io_dtype, workspace,
                             workspace_bytes, opts, stream);
        // no tokens: every sequence is empty and its final state is its initial state
        ssm::ScanPlan plan;
        ssm_status st = make_plan(1, 1, dim, dstate, io_dtype, opts, &plan);
        if (st != SSM_OK) return st;
        if (delta_softplus != 0 && delta_softplus != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "delta_softplus must be 0 or 1");
        if (!h_final) return SSM_OK;
        int64_t st_b;
        if (!bytes4(nseq, dim, dstate, 4, &st_b))
            return fail(SSM_ERR_INVALID_ARGUMENT, "state size overflows");
        if (!aligned(h_final, 16) || (h0 && !aligned(h0, 16)))
            return fail(SSM_ERR_UNSUPPORTED, "h0 and h_final must be 16-byte aligned");
        if (h0 && (const void*)h0 != (const void*)h_final &&
            overlaps(region("h_final", h_final, st_b), region("h0", h0, st_b)))
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "h_final overlaps h0 (only h_final == h0 exactly is allowed)");
        const hipError_t e = ssm::launch_copy_state(h0, h_final, st_b / 4,
                                                    static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return SSM_OK;
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

ssm_status ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                                 const void* conv_state, void* y, void* conv_state_out,
                                 int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                                 int activation, ssm_dtype io_dtype, void* stream) {
    try {
        if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
            return fail(SSM_ERR_INVALID_ARGUMENT, "io_dtype %d is not SSM_F32 or SSM_BF16",
                        (int)io_dtype);
        if (batch <= 0 || seqlen <= 0 || dim <= 0 || width <= 0)
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "sizes must be >= 1 (batch=%lld seqlen=%lld dim=%lld width=%lld)",
                        (long long)batch, (long long)seqlen, (long long)dim, (long long)width);
        if (width != 4)
            return fail(SSM_ERR_UNSUPPORTED, "width=%lld: only width 4 is supported",
                        (long long)width);
        if (activation != 0 && activation != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "activation must be 0 (none) or 1 (SiLU)");
        if (!x || !weight || !y)
            return fail(SSM_ERR_INVALID_ARGUMENT, "x, weight and y are required");
        const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
        int64_t io, stb;
        if (!bytes4(batch, dim, seqlen, elem, &io) || !bytes4(batch, dim, width - 1, elem, &stb))
            return fail(SSM_ERR_INVALID_ARGUMENT, "tensor size overflows");
        struct {
            const char* name;
            const void* p;
            uintptr_t align;
        } al[] = {{"x", x, 16}, {"y", y, 16}, {"weight", weight, 16}, {"bias", bias, 4},
                  {"conv_state", conv_state, 2}, {"conv_state_out", conv_state_out, 2}};
        for (auto& a : al)
            if (a.p && !aligned(a.p, a.align))
                return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                            (unsigned)a.align);
        const Region outs[] = {region("y", y, io), region("conv_state_out", conv_state_out, stb)};
        const Region ins[] = {region("x", x, io), region("weight", weight, dim * width * 4),
                              region("bias", bias, dim * 4),
                              region("conv_state", conv_state, stb)};
        for (const Region& o : outs)
            for (const Region& r : ins)
                if (overlaps(o, r))
                    return fail(SSM_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, r.name);
        if (overlaps(outs[0], outs[1]))
            return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps conv_state_out");
        ssm::ConvParams prm{};
        prm.x = x;
        prm.w = weight;
        prm.bias = bias;
        prm.state_in = conv_state;
        prm.y = y;
        prm.state_out = conv_state_out;
        prm.rows = batch * dim;
        prm.seqlen = seqlen;
        prm.dim = dim;
        prm.silu = activation;
        prm.aligned = ((seqlen * elem) % 16) == 0;
        const hipError_t e = ssm::launch_conv1d_fwd(prm, io_dtype == SSM_BF16,
                                                    static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return SSM_OK;
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

ssm_status ssm_causal_conv1d_update(void* conv_state, const void* x, const float* weight,
                                    const float* bias, void* y, int64_t batch, int64_t dim,
                                    int64_t width, int activation, ssm_dtype io_dtype,
                                    void* stream) {
    try {
        if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
            return fail(SSM_ERR_INVALID_ARGUMENT, "io_dtype %d is not SSM_F32 or SSM_BF16",
                        (int)io_dtype);
        if (batch <= 0 || dim <= 0 || width <= 0)
            return fail(SSM_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (batch=%lld dim=%lld "
                        "width=%lld)", (long long)batch, (long long)dim, (long long)width);
        if (width != 4)
            return fail(SSM_ERR_UNSUPPORTED, "width=%lld: only width 4 is supported",
                        (long long)width);
        if (activation != 0 && activation != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "activation must be 0 (none) or 1 (SiLU)");
        if (!conv_state || !x || !weight || !y)
            return fail(SSM_ERR_INVALID_ARGUMENT, "conv_state, x, weight and y are required");
        const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
        int64_t io, stb;
        if (!bytes4(batch, dim, 1, elem, &io) || !bytes4(batch, dim, width - 1, elem, &stb))
            return fail(SSM_ERR_INVALID_ARGUMENT, "tensor size overflows");
        struct {
            const char* name;
            const void* p;
            uintptr_t align;
        } al[] = {{"x", x, 2}, {"y", y, 2}, {"weight", weight, 16}, {"bias", bias, 4},
                  {"conv_state", conv_state, 2}};
        for (auto& a : al)
            if (a.p && !aligned(a.p, a.align))
                return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                            (unsigned)a.align);
        if (elem == 4 && (!aligned(x, 4) || !aligned(y, 4) || !aligned(conv_state, 4)))
            return fail(SSM_ERR_UNSUPPORTED, "fp32 buffers must be 4-byte aligned");
        const Region outs[] = {region("y", y, io), region("conv_state", conv_state, stb)};
        const Region ins[] = {region("x", x, io), region("weight", weight, dim * width * 4),
                              region("bias", bias, dim * 4)};
        for (const Region& o : outs)
            for (const Region& r : ins)
                if (overlaps(o, r))
                    return fail(SSM_ERR_INVALID_ARGUMENT, "%s overlaps %s", o.name, r.name);
        if (overlaps(outs[0], outs[1]))
            return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps conv_state");
        ssm::ConvParams prm{};
        prm.x = x;
        prm.w = weight;
        prm.bias = bias;
        prm.y = y;
        prm.state_out = conv_state;
        prm.rows = batch * dim;
        prm.seqlen = 1;
        prm.dim = dim;
        prm.silu = activation;
        // whole groups of 8 rows use full-width accesses when every buffer is 16-byte
        // aligned (then 8 rows of x, y and state start on 16-byte boundaries)
        prm.aligned = aligned(x, 16) && aligned(y, 16) && aligned(conv_state, 16);
        const hipError_t e = ssm::launch_conv1d_update(prm, io_dtype == SSM_BF16,
                                                       static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return SSM_OK;
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

ssm_status ssm_state_update(float* state, const void* x, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z,
                            const float* delta_bias, int delta_softplus, void* y,
                            int64_t batch, int64_t dim, int64_t dstate, ssm_dtype io_dtype,
                            void* stream) {
    try {
        if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
            return fail(SSM_ERR_INVALID_ARGUMENT, "io_dtype %d is not SSM_F32 or SSM_BF16",
                        (int)io_dtype);
        if (batch <= 0 || dim <= 0 || dstate <= 0)
            return fail(SSM_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (batch=%lld dim=%lld "
                        "dstate=%lld)", (long long)batch, (long long)dim, (long long)dstate);
        if (dstate != ssm::kDState)
            return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld: only dstate=16 is supported",
                        (long long)dstate);
        if (delta_softplus != 0 && delta_softplus != 1)
            return fail(SSM_ERR_INVALID_ARGUMENT, "delta_softplus must be 0 or 1");
        if (!state || !x || !delta || !A || !B || !C || !y)
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "state, x, delta, A, B, C and y are required");
        const int64_t elem = io_dtype == SSM_BF16 ? 2 : 4;
        int64_t st_b, io;
        if (!bytes4(batch, dim, dstate, 4, &st_b) || !bytes4(batch, dim, 1, elem, &io) ||
            batch * dim * 4 >= (int64_t(1) << 40))
            return fail(SSM_ERR_INVALID_ARGUMENT, "tensor size overflows");
        struct {
            const char* name;
            const void* p;
            uintptr_t align;
        } al[] = {{"state", state, 16}, {"x", x, 16},  {"delta", delta, 16},
                  {"z", z, 16},         {"y", y, 16},  {"B", B, 16},
                  {"C", C, 16},         {"A", A, 16},  {"D", D, 4},
                  {"delta_bias", delta_bias, 4}};
        for (auto& a : al)
            if (a.p && !aligned(a.p, a.align))
                return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                            (unsigned)a.align);
        const int64_t bc = batch * dstate * elem;
        const Region ry = region("y", y, io);
        const Region rs = region("state", state, st_b);
        const Region inputs[] = {region("x", x, io),          region("delta", delta, io),
                                 region("z", z, io),          region("B", B, bc),
                                 region("C", C, bc),          region("A", A, dim * dstate * 4),
                                 region("D", D, dim * 4),     region("delta_bias", delta_bias, dim * 4)};
        for (const Region& r : inputs) {
            if (overlaps(ry, r)) return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps %s", r.name);
            if (overlaps(rs, r))
                return fail(SSM_ERR_INVALID_ARGUMENT, "state overlaps %s", r.name);
        }
        if (overlaps(ry, rs)) return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps state");

        ssm::DecodeParams prm{};
        prm.state = state;
        prm.x = x;
        prm.delta = delta;
        prm.z = z;
        prm.y = y;
        prm.A = A;
        prm.B = B;
        prm.C = C;
        prm.D = D;
        prm.bias = delta_bias;
        prm.batch = batch;
        prm.dim = dim;
        prm.softplus = delta_softplus;
        const hipError_t e = ssm::launch_state_update(prm, io_dtype == SSM_BF16,
                                                      static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return SSM_OK;
    } catch (...) {
        return fail(SSM_ERR_INVALID_ARGUMENT, "internal error (exception)");
    }
}

}  // extern "C"
