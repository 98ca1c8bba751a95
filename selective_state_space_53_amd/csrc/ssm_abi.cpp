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

// LDS bytes of one scan workgroup of cg channels (must match the kernel's arrays).
int64_t scan_lds_bytes(int cg) { return (int64_t)(10 * cg * 36 + 2 * 1024) * 4; }

int choose_group_channels(int64_t batch, int64_t dim) {
    static const int kCands[] = {96, 80, 64, 48, 32};
    const int64_t kCUs = 256, kLds = 160 * 1024;
    int best = 32;
    double best_t = 1e300;
    int64_t best_busy = -1;
    for (int cg : kCands) {
        const int64_t groups = batch * ((dim + cg - 1) / cg);
        int64_t k = kLds / scan_lds_bytes(cg);                    // workgroups per CU
        const int64_t per_cu = (groups + kCUs - 1) / kCUs;
        if (k > per_cu) k = per_cu;
        if (k < 1) k = 1;
        const int64_t rounds = (groups + kCUs * k - 1) / (kCUs * k);
        int64_t per_simd = (k * (cg / 8) + 3) / 4;               // waves on the busiest SIMD
        if (per_simd < 2) per_simd = 2;
        const double t = (double)rounds * (double)per_simd;
        const int64_t busy = groups < kCUs ? groups : kCUs;
        if (t < best_t - 1e-9 || (t < best_t + 1e-9 && busy > best_busy)) {
            best = cg;
            best_t = t;
            best_busy = busy;
        }
    }
    return best;
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
        if (req_cg != 0 && !(req_cg >= 32 && req_cg <= 96 && req_cg % 16 == 0))
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "ssm_scan_options.group_channels=%d not in {0, 32, 48, 64, 80, 96}",
                        (int)req_cg);
        if (opts->plan < 0 || opts->plan > 2)
            return fail(SSM_ERR_INVALID_ARGUMENT, "ssm_scan_options.plan=%d not in {0,1,2}",
                        (int)opts->plan);
        if (opts->chunk_len < 0 || opts->chunk_len % ssm::kTokenTile != 0)
            return fail(SSM_ERR_INVALID_ARGUMENT,
                        "ssm_scan_options.chunk_len=%lld must be a multiple of %d",
                        (long long)opts->chunk_len, ssm::kTokenTile);
        req_plan = opts->plan;
        req_chunk = opts->chunk_len;
    }
    if (batch * ((dim + 31) / 32) >= (int64_t(1) << 30))
        return fail(SSM_ERR_INVALID_ARGUMENT, "batch*dim too large");
    const int64_t lpad = (seqlen + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;

    // Channels per workgroup (single pass): the choice with the shortest estimated
    // makespan on 256 CUs. A workgroup of cg channels runs cg/8 waves; a CU holds as
    // many workgroups as its 160 KB of LDS allows; a SIMD's time is proportional to
    // the waves it holds, except that a lone wave issues at half rate (so 1 wave costs
    // as much as 2). Ties go to more busy CUs, then to larger groups.
    const int cg_single = req_cg ? req_cg : choose_group_channels(batch, dim);
    const int64_t groups_single = batch * ((dim + cg_single - 1) / cg_single);

    // Single pass when there are enough channel groups to occupy the chip, or the
    // sequence is short; otherwise cut the sequence so that groups x chunks ~ 2048.
    bool chunked;
    if (req_plan == 1)
        chunked = false;
    else if (req_plan == 2)
        chunked = true;
    else
        chunked = groups_single < 128 && seqlen >= 4096;
    const int cg = chunked ? (req_cg ? req_cg : (dim >= 96 ? 96 : 32)) : cg_single;
    const int64_t ngroups = batch * ((dim + cg - 1) / cg);
    int64_t chunk_len = seqlen, nchunks = 1;
    if (chunked) {
        chunk_len = req_chunk;
        if (chunk_len == 0) {
            int64_t k = (2048 + ngroups - 1) / ngroups;
            if (k < 2) k = 2;
            chunk_len = (seqlen + k - 1) / k;
            chunk_len = (chunk_len + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;
        }
        nchunks = (seqlen + chunk_len - 1) / chunk_len;
        if (nchunks <= 1) {
            nchunks = 1;
            chunk_len = seqlen;
        }
    }
    if (ngroups * nchunks >= (int64_t(1) << 31))
        return fail(SSM_ERR_INVALID_ARGUMENT, "too many chunks (%lld)", (long long)nchunks);
    int64_t bcq_bytes, st_bytes = 0, sum_bytes = 0;
    if (!bytes4(batch, lpad, 4 * 8, 4, &bcq_bytes))
        return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
    if (nchunks > 1) {
        if (!bytes4(batch * dim, nchunks, ssm::kDState, 4, &st_bytes) ||
            !bytes4(batch * dim, nchunks, 1, 4, &sum_bytes))
            return fail(SSM_ERR_INVALID_ARGUMENT, "workspace size overflows");
    }
    plan->group_channels = cg;
    plan->ngroups = ngroups;
    plan->nchunks = (int)nchunks;
    plan->chunk_len = chunk_len;
    plan->ws_bcq = 0;
    plan->ws_state = align_up((size_t)bcq_bytes, 256);
    plan->ws_sum = align_up(plan->ws_state + (size_t)st_bytes, 256);
    plan->ws_total = align_up(plan->ws_sum + (size_t)sum_bytes, 256);
    return SSM_OK;
}

}  // namespace

extern "C" {

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
        ssm::ScanPlan plan;
        ssm_status st = make_plan(batch, seqlen, dim, dstate, io_dtype, opts, &plan);
        if (st != SSM_OK) return st;
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
        const int64_t st_b = batch * dim * dstate * 4;
        struct {
            const char* name;
            const void* p;
            uintptr_t align;
        } al[] = {{"x", x, 16},       {"delta", delta, 16}, {"z", z, 16},
                  {"y", y, 16},       {"B", B, 16},         {"C", C, 16},
                  {"h0", h0, 16},     {"h_final", h_final, 16},
                  {"A", A, 16},       {"D", D, 4},          {"delta_bias", delta_bias, 4},
                  {"workspace", workspace, 16}};
        for (auto& a : al)
            if (a.p && !aligned(a.p, a.align))
                return fail(SSM_ERR_UNSUPPORTED, "%s=%p is not %u-byte aligned", a.name, a.p,
                            (unsigned)a.align);
        if (plan.ws_total > 0 && (!workspace || workspace_bytes < plan.ws_total))
            return fail(SSM_ERR_WORKSPACE_TOO_SMALL,
                        "workspace needs %zu bytes (got %zu at %p)", plan.ws_total,
                        workspace_bytes, workspace);
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
                                 region("h0", h0, st_b)};
        for (const Region& r : inputs) {
            if (overlaps(ry, r))
                return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps %s", r.name);
            if (overlaps(rws, r))
                return fail(SSM_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
            if (h_final && overlaps(rhf, r)) {
                const bool same_h0 = (r.name == inputs[8].name) && (const void*)h_final == h0;
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
        prm.batch = batch;
        prm.seqlen = seqlen;
        prm.dim = dim;
        prm.lpad = (seqlen + ssm::kTokenTile - 1) / ssm::kTokenTile * ssm::kTokenTile;
        prm.chunk_len = plan.chunk_len;
        prm.nchunks = plan.nchunks;
        prm.groups_per_batch =
            (int32_t)((dim + plan.group_channels - 1) / plan.group_channels);
        prm.ngroups = (int32_t)(batch * prm.groups_per_batch);
        prm.chunk_offset = 0;
        prm.softplus = delta_softplus;
        prm.aligned = ((seqlen * elem) % 16) == 0;
        if (getenv("SSMSCAN_LOG"))
            fprintf(stderr,
                    "[ssmscan] scan b=%lld L=%lld d=%lld %s: %s, %d channels/group, %lld "
                    "groups, chunks=%d x %lld\n",
                    (long long)batch, (long long)seqlen, (long long)dim,
                    io_dtype == SSM_BF16 ? "bf16" : "f32",
                    plan.nchunks > 1 ? "chunked" : "single pass", plan.group_channels,
                    (long long)plan.ngroups, plan.nchunks, (long long)plan.chunk_len);
        hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->timing_begin) : nullptr;
        hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->timing_end) : nullptr;
        const hipError_t e = ssm::launch_scan(plan, prm, B, C, io_dtype == SSM_BF16,
                                              static_cast<hipStream_t>(stream), ev0, ev1);
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
