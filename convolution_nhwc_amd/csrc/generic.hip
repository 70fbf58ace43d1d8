// Plain one-output-per-lane forward and dgrad kernels for problems no tuned
// kernel accepts (channel counts that are not multiples of 8, strides above 4,
// depthwise shapes outside the depthwise kernels' limits).  fp32 accumulation,
// one RNE rounding per output; correct for every valid descriptor, not fast.
#include "device.h"
#include "internal.h"

namespace cnhwc {
namespace {

struct GenArgs {
    const unsigned short* in;
    const unsigned short* w;
    unsigned short* out;
    int64_t total;
    int N, H, W, C, K, R, S, stride, pad_h, pad_w, Ho, Wo, Cg, Kg;
};

template <typename T>
__global__ __launch_bounds__(256) void fwd_generic_kernel(const GenArgs a) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= a.total) return;
    const int k = int(i % a.K);
    int64_t pix = i / a.K;
    const int wo = int(pix % a.Wo);
    pix /= a.Wo;
    const int ho = int(pix % a.Ho);
    const int n = int(pix / a.Ho);
    const int g = k / a.Kg;
    float acc = 0.f;
    for (int r = 0; r < a.R; ++r) {
        const int h = ho * a.stride - a.pad_h + r;
        if (h < 0 || h >= a.H) continue;
        for (int t = 0; t < a.S; ++t) {
            const int w = wo * a.stride - a.pad_w + t;
            if (w < 0 || w >= a.W) continue;
            const unsigned short* xp = a.in + ((int64_t(n) * a.H + h) * a.W + w) * a.C + g * a.Cg;
            const unsigned short* wp = a.w + ((int64_t(k) * a.R + r) * a.S + t) * a.Cg;
            for (int j = 0; j < a.Cg; ++j) acc += to_f32<T>(xp[j]) * to_f32<T>(wp[j]);
        }
    }
    a.out[i] = pack1<T>(acc);
}

template <typename T>
__global__ __launch_bounds__(256) void dgrad_generic_kernel(const GenArgs a) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= a.total) return;
    const int c = int(i % a.C);
    int64_t pix = i / a.C;
    const int w = int(pix % a.W);
    pix /= a.W;
    const int h = int(pix % a.H);
    const int n = int(pix / a.H);
    const int g = c / a.Cg, j = c - g * a.Cg;
    float acc = 0.f;
    for (int r = 0; r < a.R; ++r) {
        const int u = h + a.pad_h - r;
        if (u < 0 || u % a.stride != 0 || u / a.stride >= a.Ho) continue;
        for (int t = 0; t < a.S; ++t) {
            const int v = w + a.pad_w - t;
            if (v < 0 || v % a.stride != 0 || v / a.stride >= a.Wo) continue;
            const unsigned short* dyp =
                a.in + ((int64_t(n) * a.Ho + u / a.stride) * a.Wo + v / a.stride) * a.K + g * a.Kg;
            for (int kk = 0; kk < a.Kg; ++kk) {
                const int64_t widx = ((int64_t(g * a.Kg + kk) * a.R + r) * a.S + t) * a.Cg + j;
                acc += to_f32<T>(dyp[kk]) * to_f32<T>(a.w[widx]);
            }
        }
    }
    a.out[i] = pack1<T>(acc);
}

GenArgs make_args(const Prob& p, const void* in, const void* w, void* out, int64_t total) {
    GenArgs a;
    a.in = static_cast<const unsigned short*>(in);
    a.w = static_cast<const unsigned short*>(w);
    a.out = static_cast<unsigned short*>(out);
    a.total = total;
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg);
    return a;
}

}  // namespace

int launch_fwd_generic(const Prob& p, const Plan&, const void* x, const void* w, void* y,
                       hipStream_t st) {
    const int64_t total = p.n * p.ho * p.wo * p.k;
    if (total == 0) return CNHWC_OK;
    const GenArgs a = make_args(p, x, w, y, total);
    const unsigned blocks = unsigned((total + 255) / 256);
    if (p.dtype == CNHWC_BF16)
        hipLaunchKernelGGL(fwd_generic_kernel<BF16>, dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(fwd_generic_kernel<F16>, dim3(blocks), dim3(256), 0, st, a);
    return CNHWC_OK;
}

int launch_dgrad_generic(const Prob& p, const Plan&, const void* dy, const void* w, void* dx,
                         hipStream_t st) {
    const int64_t total = p.n * p.h * p.w * p.c;
    if (total == 0) return CNHWC_OK;
    const GenArgs a = make_args(p, dy, w, dx, total);
    const unsigned blocks = unsigned((total + 255) / 256);
    if (p.dtype == CNHWC_BF16)
        hipLaunchKernelGGL(dgrad_generic_kernel<BF16>, dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(dgrad_generic_kernel<F16>, dim3(blocks), dim3(256), 0, st, a);
    return CNHWC_OK;
}

}  // namespace cnhwc
