// C ABI of libcnhwc: descriptor validation, output extents, the dispatcher,
// the batch-chunk planner and the launch loop.  No device code lives here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace cnhwc {
namespace {

thread_local std::string g_err;
thread_local cnhwc_override g_ov = {0, 0, 0, 0, 0};

int fail(int status, const std::string& why) {
    g_err = why;
    return status;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

// Checks in a fixed order; the first failure is reported ("feat(rocke):
// channel-packed and large-filter depthwise dgrad", C++ engine: validators
// refuse with ordered reason text).
int validate(const cnhwc_problem* in, Prob* out) {
    if (!in) return fail(CNHWC_INVALID_ARG, "problem descriptor is NULL");
    const cnhwc_problem& q = *in;
    if (q.reserved != 0) return fail(CNHWC_INVALID_ARG, "reserved field must be 0");
    const int64_t dims[7] = {q.n, q.h, q.w, q.c, q.k, q.r, q.s};
    const char* names[7] = {"n", "h", "w", "c", "k", "r", "s"};
    for (int i = 0; i < 7; ++i) {
        if (dims[i] < 1)
            return fail(CNHWC_INVALID_ARG, std::string(names[i]) + " must be >= 1 (got " +
                                               std::to_string(dims[i]) + ")");
        if (dims[i] > kMaxDim)
            return fail(CNHWC_INVALID_ARG, std::string(names[i]) + " must be < 2^31");
    }
    if (q.stride < 1)
        return fail(CNHWC_INVALID_ARG, "stride must be >= 1 (got " + std::to_string(q.stride) + ")");
    if (q.pad_h < 0 || q.pad_w < 0)
        return fail(CNHWC_INVALID_ARG, "padding must be >= 0 (got " + std::to_string(q.pad_h) +
                                           "x" + std::to_string(q.pad_w) + ")");
    if (q.groups < 1)
        return fail(CNHWC_INVALID_ARG, "groups must be >= 1 (got " + std::to_string(q.groups) + ")");
    if (q.c % q.groups != 0 || q.k % q.groups != 0)
        return fail(CNHWC_INVALID_ARG, "c and k must be multiples of groups (c=" +
                                           std::to_string(q.c) + " k=" + std::to_string(q.k) +
                                           " groups=" + std::to_string(q.groups) + ")");
    if (q.dtype != CNHWC_F16 && q.dtype != CNHWC_BF16)
        return fail(CNHWC_INVALID_ARG, "dtype must be CNHWC_F16 or CNHWC_BF16");
    const int64_t hn = q.h + 2 * int64_t(q.pad_h) - q.r;
    const int64_t wn = q.w + 2 * int64_t(q.pad_w) - q.s;
    if (hn < 0 || wn < 0)
        return fail(CNHWC_INVALID_ARG, "filter larger than the padded input (no output pixel)");
    Prob& p = *out;
    p.n = q.n; p.h = q.h; p.w = q.w; p.c = q.c; p.k = q.k; p.r = q.r; p.s = q.s;
    p.stride = q.stride; p.pad_h = q.pad_h; p.pad_w = q.pad_w; p.groups = q.groups;
    p.dtype = q.dtype;
    p.ho = hn / q.stride + 1;
    p.wo = wn / q.stride + 1;
    p.cg = q.c / q.groups;
    p.kg = q.k / q.groups;
    // keep every element count comfortably inside int64 arithmetic
    const double elems[3] = {double(p.n) * p.h * p.w * p.c, double(p.n) * p.ho * p.wo * p.k,
                             double(p.k) * p.r * p.s * p.cg};
    for (double e : elems)
        if (e > 4.0e18) return fail(CNHWC_INVALID_ARG, "tensor element count overflows int64");
    return CNHWC_OK;
}

bool is_depthwise(const Prob& p) { return p.groups == p.c && p.groups == p.k; }

bool variant_is_dgrad(int v) {
    return v == CNHWC_VAR_DGRAD_POINTWISE || v == CNHWC_VAR_DGRAD_IGEMM ||
           v == CNHWC_VAR_DGRAD_DW_STREAM || v == CNHWC_VAR_DGRAD_DW_ROTATED ||
           v == CNHWC_VAR_DGRAD_DW_TILED || v == CNHWC_VAR_DGRAD_GENERIC || v == CNHWC_VAR_DGRAD_GROUPED ||
           v == CNHWC_VAR_DGRAD_SPLITK;
}
bool variant_is_wgrad(int v) {
    return v == CNHWC_VAR_WGRAD_GENERIC || v == CNHWC_VAR_WGRAD_POINTWISE || v == CNHWC_VAR_WGRAD_SPLITK;
}
bool wgrad_uses_ws(int v) { return v == CNHWC_VAR_WGRAD_POINTWISE || v == CNHWC_VAR_WGRAD_SPLITK; }
bool variant_is_fwd(int v) {
    return v == CNHWC_VAR_FWD_DIRECT || v == CNHWC_VAR_FWD_SPLITC ||
           v == CNHWC_VAR_FWD_GROUPED || v == CNHWC_VAR_FWD_GENERIC ||
           v == CNHWC_VAR_FWD_DW_TILED || v == CNHWC_VAR_FWD_DW_ROTATED || v == CNHWC_VAR_FWD_IGEMM;
}

const char* dt(const Prob& p) { return p.dtype == CNHWC_F16 ? "f16" : "bf16"; }

// Reason a given variant cannot run the problem ("" if it can).
std::string variant_reason(const Prob& p, int op, int v, int cpl, int split_c) {
    if (op == CNHWC_OP_DGRAD && !variant_is_dgrad(v))
        return "variant " + std::to_string(v) + " is not a dgrad kernel";
    if (op == CNHWC_OP_FWD && !variant_is_fwd(v))
        return "variant " + std::to_string(v) + " is not a forward kernel";
    if (op == CNHWC_OP_WGRAD && !variant_is_wgrad(v))
        return "variant " + std::to_string(v) + " is not a wgrad kernel";
    switch (v) {
    case CNHWC_VAR_DGRAD_POINTWISE: return dgrad_igemm_reason(p, true);
    case CNHWC_VAR_DGRAD_IGEMM: return dgrad_igemm_reason(p, false);
    case CNHWC_VAR_DGRAD_SPLITK:
        if (split_c < 2) return "split-K dgrad needs at least 2 reduction splits";
        return dgrad_igemm_reason(p, false);
    case CNHWC_VAR_DGRAD_DW_STREAM: return dw_stream_reason(p, cpl);
    case CNHWC_VAR_DGRAD_DW_ROTATED: return dw_rotated_reason(p);
    case CNHWC_VAR_DGRAD_DW_TILED: return dw_tiled_reason(p);
    case CNHWC_VAR_DGRAD_GROUPED: return dgrad_grouped_reason(p);
    case CNHWC_VAR_FWD_DIRECT: return fwd_direct_reason(p, 1);
    case CNHWC_VAR_FWD_SPLITC: return fwd_direct_reason(p, split_c);
    case CNHWC_VAR_FWD_GROUPED: return fwd_grouped_reason(p);
    case CNHWC_VAR_FWD_IGEMM: return fwd_igemm_reason(p);
    case CNHWC_VAR_FWD_DW_TILED: return fwd_dw_tiled_reason(p);
    case CNHWC_VAR_FWD_DW_ROTATED: return fwd_dw_rotated_reason(p);
    case CNHWC_VAR_WGRAD_POINTWISE: return wgrad_splitk_reason(p, true);
    case CNHWC_VAR_WGRAD_SPLITK: return wgrad_splitk_reason(p, false);
    case CNHWC_VAR_FWD_GENERIC:
    case CNHWC_VAR_DGRAD_GENERIC:
    case CNHWC_VAR_WGRAD_GENERIC: return "";
    default: return "unknown variant " + std::to_string(v);
    }
}

std::string plan_name(const Prob& p, const Plan& pl) {
    char buf[160];
    switch (pl.variant) {
    case CNHWC_VAR_DGRAD_POINTWISE:
        std::snprintf(buf, sizeof buf, "dgrad_pointwise_%s", dt(p)); break;
    case CNHWC_VAR_DGRAD_IGEMM:
        if (dgrad_persist_taken(p, pl))
            std::snprintf(buf, sizeof buf, "dgrad_persist_%s_s%d", dt(p), p.stride);
        else
            std::snprintf(buf, sizeof buf, "dgrad_igemm_%s_s%d", dt(p), p.stride);
        break;
    case CNHWC_VAR_DGRAD_SPLITK:
        if (dgrad_stream_taken(p, pl))
            std::snprintf(buf, sizeof buf, "dgrad_stream_splitk%d_%s+split_reduce", pl.split_c, dt(p));
        else
            std::snprintf(buf, sizeof buf, "dgrad_splitk%d_%s_s%d+split_reduce", pl.split_c, dt(p), p.stride);
        break;
    case CNHWC_VAR_DGRAD_DW_STREAM:
        std::snprintf(buf, sizeof buf, "dgrad_dw_stream_%s_f%lldx%lld_s%d_cpl%d", dt(p),
                      (long long)p.r, (long long)p.s, p.stride, pl.cpl); break;
    case CNHWC_VAR_DGRAD_DW_ROTATED:
        std::snprintf(buf, sizeof buf, "dgrad_dw_rot_%s_f%lldx%lld_p%dx%d", dt(p),
                      (long long)p.r, (long long)p.s, p.pad_h, p.pad_w); break;
    case CNHWC_VAR_DGRAD_DW_TILED:
        std::snprintf(buf, sizeof buf, "dgrad_dw_tiled%s_%s_f%lldx%lld",
                      dw_tiled_persist_taken(p, pl) ? "_persist" : "", dt(p), (long long)p.r,
                      (long long)p.s); break;
    case CNHWC_VAR_DGRAD_GENERIC:
        std::snprintf(buf, sizeof buf, "dgrad_generic_%s", dt(p)); break;
    case CNHWC_VAR_DGRAD_GROUPED:
        std::snprintf(buf, sizeof buf, "dgrad_grouped_merge_%s", dt(p)); break;
    case CNHWC_VAR_FWD_DIRECT:
        std::snprintf(buf, sizeof buf, "fwd_direct_%s", dt(p)); break;
    case CNHWC_VAR_FWD_SPLITC:
        if (fwd_stream_taken(p, pl))
            std::snprintf(buf, sizeof buf, "fwd_stream_splitc%d_%s+split_reduce", pl.split_c, dt(p));
        else
            std::snprintf(buf, sizeof buf, "fwd_direct_splitc%d_%s+split_reduce", pl.split_c, dt(p));
        break;
    case CNHWC_VAR_FWD_GROUPED:
        std::snprintf(buf, sizeof buf, "fwd_grouped_merge_%s", dt(p)); break;
    case CNHWC_VAR_FWD_IGEMM:
        if (fwd_pw_rows_taken(p, pl))
            std::snprintf(buf, sizeof buf, "fwd_pw_rows_%s", dt(p));
        else
            std::snprintf(buf, sizeof buf, "fwd_igemm_%s_f%lldx%lld", dt(p), (long long)p.r, (long long)p.s);
        break;
    case CNHWC_VAR_FWD_GENERIC:
        std::snprintf(buf, sizeof buf, "fwd_generic_%s", dt(p)); break;
    case CNHWC_VAR_FWD_DW_TILED:
        std::snprintf(buf, sizeof buf, "fwd_dw_tiled%s_%s_f%lldx%lld",
                      dw_tiled_persist_taken(p, pl) ? "_persist" : "", dt(p), (long long)p.r,
                      (long long)p.s); break;
    case CNHWC_VAR_FWD_DW_ROTATED:
        std::snprintf(buf, sizeof buf, "fwd_dw_rot_%s_f%lldx%lld_p%dx%d", dt(p),
                      (long long)p.r, (long long)p.s, p.pad_h, p.pad_w); break;
    case CNHWC_VAR_WGRAD_GENERIC:
        std::snprintf(buf, sizeof buf, "wgrad_generic_%s", dt(p)); break;
    case CNHWC_VAR_WGRAD_POINTWISE:
        std::snprintf(buf, sizeof buf, "wgrad_pointwise_%s+reduce", dt(p)); break;
    case CNHWC_VAR_WGRAD_SPLITK:
        std::snprintf(buf, sizeof buf, "wgrad_splitk_%s_f%lldx%lld_s%d+reduce", dt(p), (long long)p.r,
                      (long long)p.s, p.stride); break;
    default: std::snprintf(buf, sizeof buf, "none");
    }
    return buf;
}

// Shape -> kernel.  The descriptor alone decides; the override exists for tests.
int choose(const Prob& p, int op, Plan* out) {
    Plan pl;
    const cnhwc_override& ov = g_ov;
    if (op != CNHWC_OP_FWD && op != CNHWC_OP_DGRAD && op != CNHWC_OP_WGRAD)
        return fail(CNHWC_INVALID_ARG,
                    "op must be CNHWC_OP_FWD (1), CNHWC_OP_DGRAD (2) or CNHWC_OP_WGRAD (4)");
    if (ov.variant != CNHWC_VAR_AUTO) {
        pl.variant = ov.variant;
        pl.cpl = ov.cpl > 0 ? ov.cpl : (ov.variant == CNHWC_VAR_DGRAD_DW_STREAM ? dw_stream_best_cpl(p) : 0);
        pl.split_c = ov.split_c > 0 ? ov.split_c
                                    : (ov.variant == CNHWC_VAR_FWD_SPLITC ? fwd_direct_auto_split(p)
                                       : ov.variant == CNHWC_VAR_DGRAD_SPLITK ? dgrad_splitk_auto(p) : 1);
        if (ov.variant == CNHWC_VAR_FWD_SPLITC && pl.split_c < 2)
            return fail(CNHWC_UNSUPPORTED, "split-C needs at least 2 channel splits");
        std::string why = variant_reason(p, op, pl.variant, pl.cpl, pl.split_c);
        if (!why.empty()) return fail(CNHWC_UNSUPPORTED, why);
        if (pl.variant != CNHWC_VAR_FWD_SPLITC && pl.variant != CNHWC_VAR_DGRAD_SPLITK) pl.split_c = 1;
        pl.tune = ov.tune;
        pl.name = plan_name(p, pl);
        *out = pl;
        return CNHWC_OK;
    }
    std::string tried;
    auto take = [&](int v, int cpl, int split) -> bool {
        std::string why = variant_reason(p, op, v, cpl, split);
        if (!why.empty()) {
            tried += (tried.empty() ? "" : "; ") + plan_name(p, Plan{v, cpl, split, 0, 0, ""}) + ": " + why;
            return false;
        }
        pl.variant = v; pl.cpl = cpl; pl.split_c = split;
        return true;
    };
    bool ok = false;
    if (op == CNHWC_OP_WGRAD) {
        if (p.r == 1 && p.s == 1 && p.stride == 1 && p.pad_h == 0 && p.pad_w == 0)
            ok = take(CNHWC_VAR_WGRAD_POINTWISE, 0, 1);
        if (!ok) ok = take(CNHWC_VAR_WGRAD_SPLITK, 0, 1);
        if (!ok) ok = take(CNHWC_VAR_WGRAD_GENERIC, 0, 1);
    } else if (op == CNHWC_OP_DGRAD) {
        if (is_depthwise(p)) {
            const bool big = p.r > 11 || p.s > 11 || p.r != p.s || p.pad_h != p.pad_w;
            if (p.stride == 1 && big) ok = take(CNHWC_VAR_DGRAD_DW_ROTATED, 0, 1);
            if (!ok && p.stride == 1) ok = take(CNHWC_VAR_DGRAD_DW_TILED, 0, 1);
            if (!ok) {
                int cpl = ov.cpl > 0 ? ov.cpl : dw_stream_best_cpl(p);
                ok = take(CNHWC_VAR_DGRAD_DW_STREAM, cpl > 0 ? cpl : 1, 1);
            }
            if (!ok && p.stride == 1) ok = take(CNHWC_VAR_DGRAD_DW_ROTATED, 0, 1);
        }
        if (!ok && p.groups > 1 && !is_depthwise(p) && p.stride == 1) ok = take(CNHWC_VAR_DGRAD_GROUPED, 0, 1);
        if (!ok && !is_depthwise(p)) {
            // few output tiles over a deep reduction: split the reduction
            const int split = ov.split_c > 0 ? ov.split_c : dgrad_splitk_auto(p);
            if (split > 1) ok = take(CNHWC_VAR_DGRAD_SPLITK, 0, split);
        }
        // 1x1 stride-1 unpadded: the pointwise fast path, grouped too (the
        // group's dY channels by offset, C/groups as the filter row stride)
        if (!ok && p.r == 1 && p.s == 1 && p.stride == 1 && p.pad_h == 0 && p.pad_w == 0)
            ok = take(CNHWC_VAR_DGRAD_POINTWISE, 0, 1);
        if (!ok) ok = take(CNHWC_VAR_DGRAD_IGEMM, 0, 1);
        if (!ok) ok = take(CNHWC_VAR_DGRAD_GENERIC, 0, 1);
    } else {
        if (is_depthwise(p) && p.stride == 1) {
            // same split as depthwise dgrad: small square filters on the tiled
            // kernel, large or non-square ones on the rotated-filter kernel
            const bool big = p.r > 11 || p.s > 11 || p.r != p.s || p.pad_h != p.pad_w;
            if (big) ok = take(CNHWC_VAR_FWD_DW_ROTATED, 0, 1);
            if (!ok) ok = take(CNHWC_VAR_FWD_DW_TILED, 0, 1);
            if (!ok) ok = take(CNHWC_VAR_FWD_DW_ROTATED, 0, 1);
        }
        if (!ok && p.groups > 1) ok = take(CNHWC_VAR_FWD_GROUPED, 0, 1);
        if (!ok && p.groups == 1 && p.r == 1 && p.s == 1 && p.stride == 1 && p.pad_h == 0 &&
            p.pad_w == 0 && ov.split_c == 0 && fwd_direct_auto_split(p) <= 1) {
            // large pointwise maps: the dgrad kernels' pointwise path (the
            // direct window kernel measured 37.3 us against 25.5 us on the
            // 32 x 56 x 56, 64 -> 256 channel layer)
            ok = take(CNHWC_VAR_FWD_IGEMM, 0, 1);
        }
        if (!ok) {
            int split = ov.split_c > 0 ? ov.split_c : fwd_direct_auto_split(p);
            if (split > 1) ok = take(CNHWC_VAR_FWD_SPLITC, 0, split);
            if (!ok) ok = take(CNHWC_VAR_FWD_DIRECT, 0, 1);
        }
        if (!ok) ok = take(CNHWC_VAR_FWD_GENERIC, 0, 1);
    }
    if (!ok) return fail(CNHWC_UNSUPPORTED, "no kernel accepts the problem: " + tried);
    pl.tune = ov.tune;
    pl.name = plan_name(p, pl);
    *out = pl;
    return CNHWC_OK;
}

struct ChunkBytes {
    int64_t per_image_max;  // largest per-image view
    int64_t fixed;          // views that do not scale with the batch (weights)
    int64_t ws_per_image;   // workspace bytes per image
    int64_t ws_fixed;       // workspace bytes independent of the batch
};

ChunkBytes chunk_bytes(const Prob& p, int op, const Plan& pl) {
    const int64_t esz = 2;
    const int64_t act = p.h * p.w * p.c * esz;
    const int64_t out = p.ho * p.wo * p.k * esz;
    ChunkBytes b;
    b.ws_per_image = 0;
    b.ws_fixed = 0;
    if (op == CNHWC_OP_FWD && pl.variant == CNHWC_VAR_FWD_IGEMM) b.ws_fixed = fwd_igemm_workspace(p);
    if (op == CNHWC_OP_FWD && pl.variant == CNHWC_VAR_FWD_SPLITC)
        b.ws_per_image = int64_t(pl.split_c) * p.ho * p.wo * p.k * 4;
    if (op == CNHWC_OP_DGRAD && pl.variant == CNHWC_VAR_DGRAD_SPLITK)
        b.ws_per_image = int64_t(pl.split_c) * p.h * p.w * p.c * 4;
    b.per_image_max = std::max(std::max(act, out), b.ws_per_image);
    b.fixed = p.k * p.r * p.s * p.cg * esz;
    return b;
}

// The override may only lower the limit: no view may pass the kernels' 32-bit range.
int64_t limit_bytes() {
    return g_ov.chunk_limit_bytes > 0 ? std::min(g_ov.chunk_limit_bytes, kBufferLimit) : kBufferLimit;
}

// Balanced batch split: the fewest chunks that keep each per-chunk view within
// the limit, sizes floor(N/chunks) or ceil(N/chunks), larger ones first.
int plan_chunks(const Prob& p, int op, const Plan& pl, std::vector<int64_t>* counts) {
    if (op == CNHWC_OP_WGRAD && pl.variant == CNHWC_VAR_WGRAD_GENERIC) {
        // the plain kernel addresses with 64-bit pointers: one launch
        counts->assign(1, p.n);
        return CNHWC_OK;
    }
    const ChunkBytes b = chunk_bytes(p, op, pl);
    const int64_t lim = limit_bytes();
    if (b.fixed > kBufferLimit)
        return fail(CNHWC_UNSUPPORTED, "weight tensor exceeds the 32-bit buffer range (" +
                                           std::to_string(b.fixed) + " bytes)");
    if (b.per_image_max > lim)
        return fail(CNHWC_UNSUPPORTED, "one image exceeds the 32-bit buffer range (" +
                                           std::to_string(b.per_image_max) + " bytes per image)");
    const int64_t max_per = lim / b.per_image_max;
    const int64_t chunks = (p.n + max_per - 1) / max_per;
    const int64_t base = p.n / chunks, extra = p.n % chunks;
    counts->clear();
    for (int64_t i = 0; i < chunks; ++i) counts->push_back(base + (i < extra ? 1 : 0));
    return CNHWC_OK;
}

int check_ptr(const void* ptr, const char* what) {
    if (!ptr) return fail(CNHWC_INVALID_ARG, std::string(what) + " is NULL");
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
        return fail(CNHWC_MISALIGNED, std::string(what) + " is not 16-byte aligned");
    return CNHWC_OK;
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + uintptr_t(nb) && y < x + uintptr_t(na);
}

int run(const cnhwc_problem* prob, int op, const void* in, const void* w, void* out, void* ws,
        size_t ws_bytes, void* stream) {
    Prob p;
    int st = validate(prob, &p);
    if (st) return st;
    Plan pl;
    if ((st = choose(p, op, &pl))) return st;
    const char* in_name = op == CNHWC_OP_FWD ? "x" : "dy";
    const char* out_name = op == CNHWC_OP_FWD ? "y" : "dx";
    if ((st = check_ptr(in, in_name))) return st;
    if ((st = check_ptr(w, "w"))) return st;
    if ((st = check_ptr(out, out_name))) return st;
    const int64_t act_bytes = p.n * p.h * p.w * p.c * 2;
    const int64_t res_bytes = p.n * p.ho * p.wo * p.k * 2;
    const int64_t in_bytes = op == CNHWC_OP_FWD ? act_bytes : res_bytes;
    const int64_t out_bytes = op == CNHWC_OP_FWD ? res_bytes : act_bytes;
    const int64_t w_bytes = p.k * p.r * p.s * p.cg * 2;
    if (overlap(out, out_bytes, in, in_bytes) || overlap(out, out_bytes, w, w_bytes))
        return fail(CNHWC_INVALID_ARG, std::string(out_name) + " overlaps an input");
    std::vector<int64_t> counts;
    if ((st = plan_chunks(p, op, pl, &counts))) return st;
    const ChunkBytes cb = chunk_bytes(p, op, pl);
    const int64_t max_chunk = *std::max_element(counts.begin(), counts.end());
    const int64_t need_ws = cb.ws_per_image * max_chunk + cb.ws_fixed;
    if (need_ws > 0) {
        if ((st = check_ptr(ws, "ws"))) return st;
        if (int64_t(ws_bytes) < need_ws)
            return fail(CNHWC_WORKSPACE_TOO_SMALL, "workspace needs " + std::to_string(need_ws) +
                                                       " bytes, got " + std::to_string(ws_bytes));
        if (overlap(ws, need_ws, in, in_bytes) || overlap(ws, need_ws, w, w_bytes) ||
            overlap(ws, need_ws, out, out_bytes))
            return fail(CNHWC_INVALID_ARG, "workspace overlaps a tensor");
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // a stale error from earlier work must not be blamed on this call
    int64_t first = 0;
    const int64_t in_img = in_bytes / p.n, out_img = out_bytes / p.n;
    for (int64_t cnt : counts) {
        Prob pc = p;
        pc.n = cnt;
        const char* ip = static_cast<const char*>(in) + first * in_img;
        char* op_ = static_cast<char*>(out) + first * out_img;
        int rc = CNHWC_OK;
        switch (pl.variant) {
        case CNHWC_VAR_DGRAD_POINTWISE:
        case CNHWC_VAR_DGRAD_IGEMM: rc = launch_dgrad_igemm(pc, pl, ip, w, op_, nullptr, s); break;
        case CNHWC_VAR_DGRAD_SPLITK: rc = launch_dgrad_igemm(pc, pl, ip, w, op_, ws, s); break;
        case CNHWC_VAR_DGRAD_DW_STREAM: rc = launch_dgrad_dw_stream(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_DGRAD_DW_ROTATED: rc = launch_dgrad_dw_rotated(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_DGRAD_DW_TILED: rc = launch_dgrad_dw_tiled(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_DGRAD_GENERIC: rc = launch_dgrad_generic(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_DGRAD_GROUPED: rc = launch_dgrad_grouped(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_FWD_DIRECT:
        case CNHWC_VAR_FWD_SPLITC: rc = launch_fwd_direct(pc, pl, ip, w, op_, ws, s); break;
        case CNHWC_VAR_FWD_GROUPED: rc = launch_fwd_grouped(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_FWD_IGEMM: rc = launch_fwd_igemm(pc, pl, ip, w, op_, ws, s); break;
        case CNHWC_VAR_FWD_GENERIC: rc = launch_fwd_generic(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_FWD_DW_TILED: rc = launch_fwd_dw_tiled(pc, pl, ip, w, op_, s); break;
        case CNHWC_VAR_FWD_DW_ROTATED: rc = launch_fwd_dw_rotated(pc, pl, ip, w, op_, s); break;
        default: rc = CNHWC_UNSUPPORTED;
        }
        if (rc) return fail(rc, "launcher for " + pl.name + " refused the chunk");
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(CNHWC_HIP_ERROR, std::string("launch of ") + pl.name + " failed: " +
                                             hipGetErrorString(e));
        first += cnt;
    }
    g_err.clear();
    return CNHWC_OK;
}

// Split-K wgrad: pixel splits of each chunk and their total.
int64_t wgrad_total_splits(const Prob& p, const Plan& pl, const std::vector<int64_t>& counts,
                           std::vector<int>* per_chunk) {
    int64_t total = 0;
    if (per_chunk) per_chunk->clear();
    for (int64_t cnt : counts) {
        Prob pc = p;
        pc.n = cnt;
        const int s = wgrad_splits(pc, pl.tune);
        if (per_chunk) per_chunk->push_back(s);
        total += s;
    }
    return total;
}

int64_t workspace_bytes(const Prob& p, int op, const Plan& pl, const std::vector<int64_t>& counts) {
    if (op == CNHWC_OP_WGRAD)
        return wgrad_uses_ws(pl.variant) ? wgrad_total_splits(p, pl, counts, nullptr) * wgrad_split_elems(p) * 4
                                         : 0;
    const int64_t mx = *std::max_element(counts.begin(), counts.end());
    const ChunkBytes cb = chunk_bytes(p, op, pl);
    return cb.ws_per_image * mx + cb.ws_fixed;
}

int run_wgrad(const cnhwc_problem* prob, const void* x, const void* dy, void* dw, void* ws,
              size_t ws_bytes, void* stream) {
    Prob p;
    int st = validate(prob, &p);
    if (st) return st;
    Plan pl;
    if ((st = choose(p, CNHWC_OP_WGRAD, &pl))) return st;
    if ((st = check_ptr(x, "x"))) return st;
    if ((st = check_ptr(dy, "dy"))) return st;
    if ((st = check_ptr(dw, "dw"))) return st;
    const int64_t x_bytes = p.n * p.h * p.w * p.c * 2;
    const int64_t dy_bytes = p.n * p.ho * p.wo * p.k * 2;
    const int64_t w_bytes = p.k * p.r * p.s * p.cg * 2;
    if (overlap(dw, w_bytes, x, x_bytes) || overlap(dw, w_bytes, dy, dy_bytes))
        return fail(CNHWC_INVALID_ARG, "dw overlaps an input");
    std::vector<int64_t> counts;
    if ((st = plan_chunks(p, CNHWC_OP_WGRAD, pl, &counts))) return st;
    const int64_t need_ws = workspace_bytes(p, CNHWC_OP_WGRAD, pl, counts);
    if (need_ws > 0) {
        if ((st = check_ptr(ws, "ws"))) return st;
        if (int64_t(ws_bytes) < need_ws)
            return fail(CNHWC_WORKSPACE_TOO_SMALL, "workspace needs " + std::to_string(need_ws) +
                                                       " bytes, got " + std::to_string(ws_bytes));
        if (overlap(ws, need_ws, x, x_bytes) || overlap(ws, need_ws, dy, dy_bytes) ||
            overlap(ws, need_ws, dw, w_bytes))
            return fail(CNHWC_INVALID_ARG, "workspace overlaps a tensor");
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    auto launched = [&](const char* what) -> int {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(CNHWC_HIP_ERROR, std::string("launch of ") + what + " failed: " + hipGetErrorString(e));
        return CNHWC_OK;
    };
    if (pl.variant == CNHWC_VAR_WGRAD_GENERIC) {
        int rc = launch_wgrad_generic(p, x, dy, dw, s);
        if (rc) return fail(rc, "launcher for " + pl.name + " refused the problem");
        if ((rc = launched(pl.name.c_str()))) return rc;
        g_err.clear();
        return CNHWC_OK;
    }
    std::vector<int> splits;
    const int64_t total = wgrad_total_splits(p, pl, counts, &splits);
    float* wsf = static_cast<float*>(ws);
    const int64_t x_img = x_bytes / p.n, dy_img = dy_bytes / p.n;
    int64_t first = 0, split_base = 0;
    for (size_t i = 0; i < counts.size(); ++i) {
        Prob pc = p;
        pc.n = counts[i];
        const char* xp = static_cast<const char*>(x) + first * x_img;
        const char* yp = static_cast<const char*>(dy) + first * dy_img;
        int rc = launch_wgrad_splitk(pc, pl, xp, yp, wsf + split_base * wgrad_split_elems(p), splits[i], s);
        if (rc) return fail(rc, "launcher for " + pl.name + " refused the chunk");
        if ((rc = launched(pl.name.c_str()))) return rc;
        first += counts[i];
        split_base += splits[i];
    }
    int rc = launch_wgrad_reduce(p, int(total), wsf, dw, s);
    if (rc) return fail(rc, "wgrad reduce refused the problem");
    if ((rc = launched("wgrad_reduce"))) return rc;
    g_err.clear();
    return CNHWC_OK;
}

}  // namespace

int set_error(int status, const std::string& why) { return fail(status, why); }

}  // namespace cnhwc

using namespace cnhwc;

extern "C" {

int cnhwc_out_dims(const cnhwc_problem* prob, int64_t* ho, int64_t* wo) {
    Prob p;
    int st = validate(prob, &p);
    if (st) return st;
    if (ho) *ho = p.ho;
    if (wo) *wo = p.wo;
    g_err.clear();
    return CNHWC_OK;
}

int cnhwc_workspace_size(const cnhwc_problem* prob, int op, size_t* bytes) {
    Prob p;
    int st = validate(prob, &p);
    if (st) return st;
    Plan pl;
    if ((st = choose(p, op, &pl))) return st;
    std::vector<int64_t> counts;
    if ((st = plan_chunks(p, op, pl, &counts))) return st;
    if (bytes) *bytes = size_t(workspace_bytes(p, op, pl, counts));
    g_err.clear();
    return CNHWC_OK;
}

int cnhwc_plan(const cnhwc_problem* prob, int op, char* name, size_t cap, int32_t* variant) {
    Prob p;
    int st = validate(prob, &p);
    if (st) return st;
    Plan pl;
    if ((st = choose(p, op, &pl))) return st;
    if (name && cap > 0) {
        std::strncpy(name, pl.name.c_str(), cap - 1);
        name[cap - 1] = '\0';
    }
    if (variant) *variant = pl.variant;
    g_err.clear();
    return CNHWC_OK;
}

int cnhwc_chunk_plan(const cnhwc_problem* prob, int op, int64_t* counts, int64_t cap,
                     int64_t* nchunks) {
    Prob p;
    int st = validate(prob, &p);
    if (st) return st;
    Plan pl;
    if ((st = choose(p, op, &pl))) return st;
    std::vector<int64_t> c;
    if ((st = plan_chunks(p, op, pl, &c))) return st;
    if (nchunks) *nchunks = int64_t(c.size());
    for (int64_t i = 0; counts && i < cap && i < int64_t(c.size()); ++i) counts[i] = c[i];
    g_err.clear();
    return CNHWC_OK;
}

int cnhwc_fwd(const cnhwc_problem* prob, const void* x, const void* w, void* y, void* ws,
              size_t ws_bytes, void* hip_stream) {
    return run(prob, CNHWC_OP_FWD, x, w, y, ws, ws_bytes, hip_stream);
}

int cnhwc_dgrad(const cnhwc_problem* prob, const void* dy, const void* w, void* dx, void* ws,
                size_t ws_bytes, void* hip_stream) {
    return run(prob, CNHWC_OP_DGRAD, dy, w, dx, ws, ws_bytes, hip_stream);
}

int cnhwc_wgrad(const cnhwc_problem* prob, const void* x, const void* dy, void* dw, void* ws,
                size_t ws_bytes, void* hip_stream) {
    return run_wgrad(prob, x, dy, dw, ws, ws_bytes, hip_stream);
}

const char* cnhwc_last_error(void) { return g_err.c_str(); }

int cnhwc_set_override(const cnhwc_override* ov) {
    if (!ov) {
        g_ov = cnhwc_override{0, 0, 0, 0, 0};
        return CNHWC_OK;
    }
    if (ov->cpl != 0 && ov->cpl != 1 && ov->cpl != 2 && ov->cpl != 4 && ov->cpl != 8)
        return fail(CNHWC_INVALID_ARG, "cpl must be 1, 2, 4 or 8 (got " + std::to_string(ov->cpl) + ")");
    if (ov->split_c < 0) return fail(CNHWC_INVALID_ARG, "split_c must be >= 0");
    if (ov->tune < 0) return fail(CNHWC_INVALID_ARG, "tune must be >= 0");
    if (ov->chunk_limit_bytes < 0) return fail(CNHWC_INVALID_ARG, "chunk_limit_bytes must be >= 0");
    g_ov = *ov;
    g_err.clear();
    return CNHWC_OK;
}

}  // extern "C"
