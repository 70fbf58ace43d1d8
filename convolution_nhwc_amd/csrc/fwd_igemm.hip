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

#include <algorithm>

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

// ---------------------------------------------------------------------------
// Pointwise forward (1x1, stride 1, unpadded, one group) for up to 64 input
// channels and up to 256 output channels: y[m][k] = sum_c x[m][c] W[k][c],
// a GEMM over the flattened pixels m, read straight from the filter as stored
// (no transform pass).  Built around HBM access, like the row-streamed
// pointwise dgrad: the filter sits in every wave's registers as MFMA operand
// fragments (lane = output channel row, 8 consecutive input channels), each
// wave walks its own 16-pixel blocks (no barriers after the set-up) with one
// 16-byte load a lane per 32 input channels straight into the pixel operand,
// the next block's loads in flight while one is multiplied.  A finished block
// (16 pixels x K channels, contiguous in y) is rounded into the wave's own
// LDS staging area (16-byte chunks XOR-ed by pixel row) and written back as
// whole contiguous 1 KiB stores.  Each output runs the ring kernel's chain
// (ascending 32-deep MFMA steps, the same lane / k assignment), so the two
// paths give the same bits.
struct FpArgs {
    const void* x;
    const void* w;
    void* y;
    uint32_t x_bytes, w_bytes, y_bytes;
    int M, C, K;
};

constexpr int kFpThreads = 256;   // 4 waves; two blocks per CU

template <typename T, int KT, int CS>   // KT = K / 16 output tiles, CS = C / 32 input steps
__global__ __launch_bounds__(kFpThreads, 2) void fwd_pw_rows_kernel(const FpArgs a) {
    constexpr int ROWB = KT * 32;                   // bytes of one output pixel
    constexpr int CH = KT * 2;                      // its 16-byte chunks
    constexpr int SWM = (CH < 16 ? CH : 16) - 1;    // chunk swizzle mask
    constexpr int STG = 16 * ROWB;                  // a wave's staging area
    constexpr int WROW = CS * 64;                   // bytes of one filter row
    constexpr int WB = KT * 16 * WROW;              // the filter
    static_assert(STG % 1024 == 0, "whole 1 KiB stores");
    __shared__ __attribute__((aligned(16))) unsigned char lds[WB + 4 * STG];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frow = lane & 15, fgrp = lane >> 4;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);

    // ---- the filter (K rows of C channels, as stored) -> LDS -> registers:
    // fragment (j, s): lane = output channel j*16 + frow, input channels
    // s*32 + fgrp*8 .. +7 ----
    for (int q = tid; q < WB / 16; q += kFpThreads)
        *reinterpret_cast<i32x4*>(lds + q * 16) = buf_load16(rw, uint32_t(q * 16));
    __syncthreads();
    i32x4 wf[KT][CS];
#pragma unroll
    for (int j = 0; j < KT; ++j)
#pragma unroll
        for (int s = 0; s < CS; ++s)
            wf[j][s] = *reinterpret_cast<const i32x4*>(lds + (j * 16 + frow) * WROW + (s * 32 + fgrp * 8) * 2);

    unsigned char* const sg = lds + WB + wave * STG;
    const int nblk = (a.M + 15) / 16;
    const int gw = blockIdx.x * 4 + wave, gws = gridDim.x * 4;
    // pixel operand of block b: lane = pixel b*16 + frow, channels s*32 + fgrp*8 .. +7
    auto load_x = [&](int b, i32x4 (&xf)[CS]) {
        const int m = b * 16 + frow;
#pragma unroll
        for (int s = 0; s < CS; ++s)
            xf[s] = buf_load16(rx, b < nblk && m < a.M ? uint32_t((m * a.C + s * 32 + fgrp * 8) * 2) : kOob);
    };
    auto block = [&](int b, const i32x4 (&xf)[CS]) {
        f32x4 acc[KT];
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            acc[j] = mfma16x16x32<T>(wf[j][0], xf[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int s = 1; s < CS; ++s) acc[j] = mfma16x16x32<T>(wf[j][s], xf[s], acc[j]);
        }
        // lane: output channels j*16 + fgrp*4 .. +3 of pixel frow
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const i32x2 v = {int(pack2<T>(acc[j][0], acc[j][1])), int(pack2<T>(acc[j][2], acc[j][3]))};
            const int chunk = (j * 2 + (fgrp >> 1)) ^ (frow & SWM);
            *reinterpret_cast<i32x2*>(sg + frow * ROWB + chunk * 16 + (fgrp & 1) * 8) = v;
        }
        // the block's rows are contiguous in y: chunk e of the block at byte b*STG + 16e
#pragma unroll
        for (int q = 0; q < STG / 1024; ++q) {
            const int e = q * 64 + lane;
            const int r = e / CH, cc = e % CH;
            const i32x4 v = *reinterpret_cast<const i32x4*>(sg + r * ROWB + ((cc ^ (r & SWM)) << 4));
            const int m = b * 16 + r;
            buf_store16(v, ry, m < a.M ? uint32_t(b * STG + e * 16) : kOob);
        }
    };
    i32x4 x0[CS], x1[CS];
    load_x(gw, x0);
#pragma unroll 1
    for (int b = gw; b < nblk; b += 2 * gws) {
        load_x(b + gws, x1);
        block(b, x0);
        if (b + gws >= nblk) break;
        load_x(b + 2 * gws, x0);
        block(b + gws, x1);
    }
}

template <typename T, int KT>
void launch_fp_kt(int cs, const FpArgs& a, int grid, hipStream_t st) {
    if (cs == 1) hipLaunchKernelGGL((fwd_pw_rows_kernel<T, KT, 1>), dim3(grid), dim3(kFpThreads), 0, st, a);
    else hipLaunchKernelGGL((fwd_pw_rows_kernel<T, KT, 2>), dim3(grid), dim3(kFpThreads), 0, st, a);
}

template <typename T>
void launch_fp(int kt, int cs, const FpArgs& a, int grid, hipStream_t st) {
    if (kt == 4) launch_fp_kt<T, 4>(cs, a, grid, st);
    else if (kt == 8) launch_fp_kt<T, 8>(cs, a, grid, st);
    else launch_fp_kt<T, 16>(cs, a, grid, st);
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

// The pointwise row kernel takes 1x1 stride-1 unpadded single-group forwards
// with C in {32, 64} and K in {64, 128, 256} (tune 1 keeps the transform and
// the dgrad kernels).
bool fwd_pw_rows_taken(const Prob& p, const Plan& pl) {
    return pl.variant == CNHWC_VAR_FWD_IGEMM && pl.tune != 1 && p.r == 1 && p.s == 1 && p.stride == 1 &&
           p.pad_h == 0 && p.pad_w == 0 && p.groups == 1 && (p.c == 32 || p.c == 64) &&
           (p.k == 64 || p.k == 128 || p.k == 256);
}

int launch_fwd_igemm(const Prob& p, const Plan& pl, const void* x, const void* w, void* y, void* ws,
                     hipStream_t st) {
    if (fwd_pw_rows_taken(p, pl)) {
        FpArgs a{};
        a.x = x; a.w = w; a.y = y;
        a.M = int(p.n * p.h * p.w);
        a.C = int(p.c); a.K = int(p.k);
        a.x_bytes = uint32_t(int64_t(a.M) * a.C * 2);
        a.w_bytes = uint32_t(int64_t(a.K) * a.C * 2);
        a.y_bytes = uint32_t(int64_t(a.M) * a.K * 2);
        if (a.M <= 0) return CNHWC_OK;
        const int64_t waves = (int64_t(a.M) + 15) / 16;
        const int grid = int(std::min<int64_t>(2 * kNumCUs, (waves + 3) / 4));
        const int kt = a.K / 16, cs = a.C / 32;
        if (p.dtype == CNHWC_BF16) launch_fp<BF16>(kt, cs, a, grid, st);
        else launch_fp<F16>(kt, cs, a, grid, st);
        return CNHWC_OK;
    }
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
