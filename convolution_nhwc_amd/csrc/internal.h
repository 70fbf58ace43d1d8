// Host-side internals shared by the C ABI (host.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/cnhwc.h"

namespace cnhwc {

// A validated problem with its derived extents.
struct Prob {
    int64_t n, h, w, c, k, r, s;
    int64_t ho, wo;   // output rows / columns (floor formula)
    int64_t cg, kg;   // channels per group of x and of y
    int32_t stride, pad_h, pad_w, groups;
    int32_t dtype;    // CNHWC_F16 / CNHWC_BF16
};

// The dispatcher's decision for one pass.
struct Plan {
    int32_t variant = CNHWC_VAR_AUTO;
    int32_t cpl = 0;      // depthwise channels per lane
    int32_t split_c = 1;  // channel splits of the split-C forward
    int32_t tile = 0;     // variant-specific tile selector
    int32_t tune = 0;     // test-only launch-shape knob (0 = automatic)
    std::string name;
};

// Number of compute units the kernels size their grids for (MI355X: 256).
constexpr int kNumCUs = 256;

// Per-view byte limit of the kernels' 32-bit buffer addressing.
constexpr int64_t kBufferLimit = (int64_t(1) << 31) - 1;

// ---- launchers (one batch chunk each; p.n is the chunk's batch) -------------
// Each returns 0 on success or a CNHWC_* status; launch errors are reported by
// the caller through hipGetLastError.
// Implicit-GEMM dgrad (pointwise fast path, general strided, and split-K:
// fp32 partials of pl.split_c reduction splits into ws[split][N*H*W][C], then
// the split reduce pass into dx).
int launch_dgrad_igemm(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                       void* ws, hipStream_t st);
// Split-K dgrad: automatic number of reduction splits (1 = do not split).
int dgrad_splitk_auto(const Prob& p);
// Forward (stride 1, groups 1) as the dgrad of the rotated, transposed filter
// on the implicit-GEMM dgrad kernels; ws receives the transformed filter
// (fwd_igemm_workspace bytes, independent of the batch).
int launch_fwd_igemm(const Prob& p, const Plan& pl, const void* x, const void* w, void* y, void* ws,
                     hipStream_t st);
int64_t fwd_igemm_workspace(const Prob& p);
std::string fwd_igemm_reason(const Prob& p);
int launch_dgrad_dw_stream(const Prob& p, const Plan& pl, const void* dy, const void* w,
                           void* dx, hipStream_t st);
int launch_dgrad_dw_rotated(const Prob& p, const Plan& pl, const void* dy, const void* w,
                            void* dx, hipStream_t st);
int launch_dgrad_dw_tiled(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                          hipStream_t st);
int launch_dgrad_generic(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                         hipStream_t st);
int launch_fwd_direct(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                      void* ws, hipStream_t st);
int launch_fwd_window(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                      void* ws, hipStream_t st);
// Split-C forward for small output maps (N*Ho*Wo <= 448) that streams the
// filter once: its split count (0 if it does not apply), acceptance and launch
// (main pass + the split reduce).
int fwd_stream_splits(const Prob& p);
std::string fwd_stream_reason(const Prob& p, int splits);
int launch_fwd_stream(const Prob& p, const Plan& pl, const void* x, const void* w, void* y, void* ws,
                      hipStream_t st);
// Whether the split-C forward of this plan runs on the filter-streaming kernel.
bool fwd_stream_taken(const Prob& p, const Plan& pl);
// Split-K dgrad (stride 1, groups 1) on the filter-streaming kernel: its split
// count (0 if it does not apply), acceptance, whether a plan takes it, launch
// (main pass + the split reduce).
// Whether the implicit-GEMM forward plan runs the pointwise row kernel
// (fwd_igemm.hip: 1x1 stride-1 unpadded single-group, C 32/64, K 64/128/256).
bool fwd_pw_rows_taken(const Prob& p, const Plan& pl);
// Strided dgrad on the persistent 8-wave kernel (dgrad_persist.hip): the
// reason it cannot run a problem ("" if it can), whether the implicit-GEMM plan
// takes it (automatic choice for stride >= 2, or tune 5), and its launch.
std::string dgrad_persist_reason(const Prob& p);
bool dgrad_persist_taken(const Prob& p, const Plan& pl);
int launch_dgrad_persist(const Prob& p, const void* dy, const void* w, void* dx, hipStream_t st);
int dgrad_stream_splits(const Prob& p);
std::string dgrad_stream_reason(const Prob& p, int splits);
bool dgrad_stream_taken(const Prob& p, const Plan& pl);
int launch_dgrad_stream(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx, void* ws,
                        hipStream_t st);
// Second pass of split-C: y = round(sum over splits of ws[split]), ascending.
int launch_split_reduce(const Prob& p, int splits, const void* ws, void* y, hipStream_t st);
int launch_fwd_grouped(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                       hipStream_t st);
int launch_fwd_generic(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                       hipStream_t st);
// Grouped dgrad, stride 1, small groups merged: the whole-row grouped kernel.
int launch_dgrad_grouped(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                         hipStream_t st);
// Depthwise forward, stride 1, on the depthwise dgrad kernels (rotation identity).
int launch_fwd_dw_tiled(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                        hipStream_t st);
int launch_fwd_dw_rotated(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                          hipStream_t st);

// Weight gradient.  Split-K MFMA kernel (one chunk: fp32 partials of `splits`
// pixel splits into ws[split][K][R][S][Cg]), the reduce pass over all splits
// of all chunks, and the plain kernel (whole batch, 64-bit addressing).
int launch_wgrad_splitk(const Prob& p, const Plan& pl, const void* x, const void* dy, float* ws,
                        int splits, hipStream_t st);
int launch_wgrad_reduce(const Prob& p, int splits, const float* ws, void* dw, hipStream_t st);
int launch_wgrad_generic(const Prob& p, const void* x, const void* dy, void* dw, hipStream_t st);
// Pixel splits of one chunk (tune > 0 forces that many) and the elements of
// one split's partial tile (K*R*S*Cg).
int wgrad_splits(const Prob& p, int tune);
int64_t wgrad_split_elems(const Prob& p);

// Records `why` as this thread's cnhwc_last_error() reason and returns status.
int set_error(int status, const std::string& why);

// ---- per-variant acceptance (empty string = accepted, else the reason) ------
std::string dgrad_igemm_reason(const Prob& p, bool pointwise);
std::string dw_stream_reason(const Prob& p, int cpl);
std::string dw_rotated_reason(const Prob& p);
std::string dw_tiled_reason(const Prob& p);
// the LDS-tiled depthwise variant (dgrad or forward) runs the persistent 7x7 kernel
bool dw_tiled_persist_taken(const Prob& p, const Plan& pl);
bool dw_tiled_persist_applies(const Prob& p, int tune);
std::string fwd_dw_tiled_reason(const Prob& p);
std::string dgrad_grouped_reason(const Prob& p);
std::string fwd_dw_rotated_reason(const Prob& p);
std::string fwd_direct_reason(const Prob& p, int split_c);
std::string wgrad_splitk_reason(const Prob& p, bool pointwise);
std::string fwd_grouped_reason(const Prob& p);
std::string fwd_window_reason(const Prob& p, int split_c);
int fwd_window_auto_split(const Prob& p);

// Depthwise row-streaming: the largest channels-per-lane the kernel set has an
// instance for at this filter/stride (0 if none).
int dw_stream_best_cpl(const Prob& p);
// Split-C forward: tile grid size and the automatic split count.
int64_t fwd_direct_tiles(const Prob& p);
int fwd_direct_auto_split(const Prob& p);
int fwd_direct_channel_chunk();

}  // namespace cnhwc
