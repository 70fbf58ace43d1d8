// Forward convolution (stride 1) on the implicit-GEMM dgrad kernels.
//
// Stride-1 dgrad is a correlation of dY with the filter rotated by 180 degrees
// at padding R-1-pad ("feat(rocke): channel-packed and large-filter depthwise
// dgrad", Rotated-filter dgrad); read the other way, a stride-1 forward
//
//   y[n, ho, wo, k] = sum_{r, t, c} x[n, ho - pad_h + r, wo - pad_w + t, c] * W[k, r, t, c]
//
// is the dgrad of a problem whose dY is x (K_d = C channels, extents H x W),
// whose dX is y (C_d = K channels, extents Ho x Wo), with padding
// (R-1-pad_h, S-1-pad_w) and filter
//
//   W_d[c][r'][t'][k] = W[k][R-1-r'][S-1-t'][c]
//
// (dgrad reads dY row u = h + pad_d - r', i.e. x row ho - pad_h + (R-1-r')).
// A transform pass writes W_d into the caller's workspace; the dgrad
// dispatcher's kernels (dY-window, ring, pointwise) then run unchanged.  This
// is the implicit-GEMM forward for large maps, where the direct window
// kernel's halo grows with the map and its tiles stay small.
#include "device.h"
#include "internal.h"

#include <string>

namespace cnhwc {
namespace {

// W_d[c][r'][t'][k] = W[k][R-1-r'][S-1-t'][c]: one output element per lane
// (writes coalesced along k).
__global__ __launch_bounds__(256) void fwd_filter_transform_kernel(const unsigned short* __restrict__ w,
                                                                   unsigned short* __restrict__ wd,
                                                                   int K, int R, int S, int C,
                                                                   int64_t total) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int k = int(i % K);
    int64_t q = i / K;
    const int t = int(q % S);
    q /= S;
    const int r = int(q % R);
    const int c = int(q / R);
    wd[i] = w[((int64_t(k) * R + (R - 1 - r)) * S + (S - 1 - t)) * C + c];
}

// The dgrad problem a stride-1 forward problem maps to (see above).
Prob as_dgrad(const Prob& p) {
    Prob d = p;
    d.h = p.ho; d.w = p.wo;          // dX_d = y
    d.ho = p.h; d.wo = p.w;          // dY_d = x
    d.c = p.k; d.k = p.c;
    d.cg = p.k; d.kg = p.c;
    d.pad_h = int32_t(p.r - 1 - p.pad_h);
    d.pad_w = int32_t(p.s - 1 - p.pad_w);
    return d;
}

bool pointwise_d(const Prob& d) {
    return d.r == 1 && d.s == 1 && d.stride == 1 && d.pad_h == 0 && d.pad_w == 0 && d.groups == 1;
}

}  // namespace

std::string fwd_igemm_reason(const Prob& p) {
    if (p.groups != 1) return "implicit-GEMM forward needs groups == 1";
    if (p.stride != 1) return "implicit-GEMM forward needs stride 1";
    if (p.pad_h > p.r - 1 || p.pad_w > p.s - 1)
        return "implicit-GEMM forward needs pad_h <= R-1 and pad_w <= S-1 (rotated padding >= 0)";
    const Prob d = as_dgrad(p);
    return dgrad_igemm_reason(d, pointwise_d(d));
}

int64_t fwd_igemm_workspace(const Prob& p) { return p.k * p.r * p.s * p.c * 2; }

int launch_fwd_igemm(const Prob& p, const Plan& pl, const void* x, const void* w, void* y, void* ws,
                     hipStream_t st) {
    if (ws == nullptr) return CNHWC_UNSUPPORTED;
    const int64_t total = p.k * p.r * p.s * p.c;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > (int64_t(1) << 31) - 1) return CNHWC_UNSUPPORTED;
    hipLaunchKernelGGL(fwd_filter_transform_kernel, dim3(unsigned(blocks)), dim3(256), 0, st,
                       static_cast<const unsigned short*>(w), static_cast<unsigned short*>(ws),
                       int(p.k), int(p.r), int(p.s), int(p.c), total);
    const Prob d = as_dgrad(p);
    Plan dp = pl;
    dp.variant = pointwise_d(d) ? CNHWC_VAR_DGRAD_POINTWISE : CNHWC_VAR_DGRAD_IGEMM;
    dp.split_c = 1;
    return launch_dgrad_igemm(d, dp, x, ws, y, nullptr, st);
}

}  // namespace cnhwc
