// Weight gradient (wgrad): the derivative of the forward map with respect to
// the weight, the third convolution pass beside forward and dgrad ("perf(rocke/
// conv): add the pointwise fast path dgrad was missing", Motivation: forward
// and wgrad both special-case 1x1 convolutions).
//
//   dW[k][r][t][j] = sum over output pixels m = (n, ho, wo) of
//                    dY[m][k] * x[n, ho*s - pad_h + r, wo*s - pad_w + t, g*Cg + j],  g = k / Kg
//
// (x read as zero outside the image).  Per filter tap (r, t) this is a GEMM
// dW_tap[k][j] = sum_m dY[m][k] * X_tap[m][j] whose reduction runs over all
// N*Ho*Wo output pixels: deep and narrow, so the pixels are split across
// blocks (split-K) and each block writes an fp32 partial tile to a workspace
// [split][K][R][S][Cg]; a second pass sums the splits in a fixed order and
// rounds once (round to nearest even) to fp16 / bf16.
//
// Split-K kernel data path (gfx950): one block per (group, 128-channel k
// block, tap, j block of 64 or 128 input channels) and pixel split.  It
// streams its split 32 output pixels at a time: the dY rows (k slice) and the
// tap's input rows (j slice, gathered pixel by pixel, zero outside the image
// through the buffer range check) go global -> LDS by LDS-direct DMA into a
// four-stage ring, so three stages are in flight while one is multiplied.
// Both tiles keep pixels as rows, exactly as they lie in memory; the MFMA
// operands (eight consecutive pixels of one channel per lane) come from the
// LDS transpose read (ds_read_b64_tr_b16).  The 16-byte chunks of each row are
// XOR-swizzled by row at the source (the DMA writes LDS linearly) so that the
// 16 rows one transpose read touches fall on distinct bank groups.  The MFMA
// computes the transposed product (j x k), so each lane ends with four
// consecutive j of one k: one 16-byte fp32 store per tile fragment.
//
// The 1x1 stride-1 unpadded case is the same kernel with the gather dropped:
// the input row of output pixel m is row m itself (offset m*C + g*Cg + j, as
// the fast-path commit on the first page states for the pointwise offsets),
// so no division by Ho*Wo and Wo is made per row.  Same reduction order, same
// rounding: bit-identical to the general kernel on the same problem.
//
// A plain one-weight-per-lane kernel covers every other valid problem.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>

namespace cnhwc {
namespace {

constexpr int kWBM = 32;         // output pixels per stage (one MFMA depth)

// Block shapes: NW waves over a (32 NW output channels k) x (BJ input channels
// j) tile, each wave 64 x 64 (or 32 x 64); NS ring stages.  4 waves: k 128,
// 4 stages, two blocks a CU; 8 waves: k 256, 3 stages (the stage offsets stay
// within the LDS immediate), two blocks a CU -- half the input-tile bytes per
// product and half the per-wave gather work for the same per-wave tile.
constexpr int wg_kb(int nw) { return 32 * nw; }
constexpr int wg_stages(int nw) { return nw == 8 ? 3 : 4; }

struct WgArgs {
    const void* x;
    const void* dy;
    float* ws;                   // this chunk's first split
    uint32_t x_bytes, dy_bytes;
    int N, H, W, C, K, R, S, stride, pad_h, pad_w, Ho, Wo, Cg, Kg;
    int P;                       // output pixels of the chunk
    int kblocks, jblocks, tiles; // per group: ceil(Kg/128), ceil(Cg/BJ); all tiles
    int splits;                  // pixel splits of the chunk
    int remap;                   // 1: deal logical blocks to XCDs in contiguous runs (any block count)
    FastDiv div_hw, div_w;       // by Ho*Wo, by Wo
    int step_ho, step_wo;        // 32 output pixels = step_ho rows + step_wo columns (32 / Wo, 32 % Wo)
    int64_t split_elems;         // K*R*S*Cg (workspace stride of one split)
};

// Source-side chunk swizzle of a stage row.  A transpose read touches rows
// 8f + 4h + i (f, i = 0..3) of one 32-byte chunk pair; the value XOR-ed into
// the chunk index spreads those 16 rows over 8 distinct pair positions (256 B
// rows) or, with 128 B rows, over 4 positions x the two row parities.
template <int CHUNKS>
__device__ inline int wswz(int row) {
    if constexpr (CHUNKS >= 16) return 2 * ((row & 3) | ((row >> 1) & 4));
    else return 2 * (((row >> 1) & 1) | ((row >> 2) & 2));
}

template <typename T, int BJ, bool PW, int NW>
__global__ __launch_bounds__(NW * 64, 2) void wgrad_splitk_kernel(const WgArgs a) {
    constexpr int kWBK = wg_kb(NW);                  // output channels (k) per block
    constexpr int kWStages = wg_stages(NW);
    constexpr int WAVES_J = BJ / 64;                 // 1 or 2
    constexpr int WAVES_K = NW / WAVES_J;
    constexpr int WJT = 4;                           // 16-wide j tiles per wave
    constexpr int WKT = kWBK / (WAVES_K * 16);       // 16-wide k tiles per wave: 2 or 4
    constexpr int XROW = BJ * 2;                     // bytes of one input row in a stage
    constexpr int XCH = BJ / 8;                      // 16-byte chunks per input row
    constexpr int YROW = kWBK * 2;                   // bytes of one dY row in a stage
    constexpr int YCH = kWBK / 8;
    constexpr int XBYTES = kWBM * XROW;
    constexpr int STAGE = XBYTES + kWBM * YROW;
    constexpr int XD = XBYTES / 1024;                // 1 KB DMAs of the input tile
    constexpr int ND = STAGE / 1024;
    constexpr int LPS = ND / NW;                     // DMAs per wave per stage
    static_assert(ND % NW == 0, "stage must split evenly over the waves");
    static_assert((kWStages - 1) * STAGE < 65536, "stage offsets fit the LDS immediate");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kWStages * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: the DMA roles below branch on it, and each wave
    // must issue exactly LPS loads per stage for the vmcnt waits to hold
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frow = lane & 15, fgrp = lane >> 4;

    // ---- block -> (split, group, k block, tap, j block) ----
    int bid = blockIdx.x;
    if (a.remap) {
        // XCD x = bid % 8 runs blocks x, x + 8, ...; give it the contiguous
        // logical run [x q + min(x, r), ...) (q + 1 blocks for x < r), so the
        // taps and j blocks of one pixel split -- which read the same dY rows
        // -- share an L2
        const int q = int(gridDim.x >> 3), rr = int(gridDim.x & 7), x = bid & 7;
        bid = x * q + min(x, rr) + (bid >> 3);
    }
    const int split = bid / a.tiles;
    int tile = bid - split * a.tiles;
    const int jb = tile % a.jblocks;
    tile /= a.jblocks;
    const int RS = a.R * a.S;
    const int tap = tile % RS;
    tile /= RS;
    const int kb = tile % a.kblocks;
    const int g = tile / a.kblocks;
    const int r = tap / a.S, t = tap - r * a.S;
    const int m_begin = int(int64_t(split) * a.P / a.splits);
    const int m_end = int(int64_t(split + 1) * a.P / a.splits);
    const int nsteps = (m_end - m_begin + kWBM - 1) / kWBM;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);

    // ---- per-lane DMA roles: DMA q = NW*d + wave covers bytes [1024q, 1024q+1024)
    // of a stage.  The first XL slots of every wave are input rows, the rest dY
    // rows, so the input gather's address arithmetic is shared by all waves ----
    constexpr int XL = XD / NW;                      // input DMAs per wave per stage
    static_assert(XD % NW == 0, "input tile must split evenly over the waves");
    int d_row[LPS];              // stage row (pixel 0..31)
    uint32_t d_chan[LPS];        // channel byte offset within the pixel, or kOob
#pragma unroll
    for (int d = 0; d < LPS; ++d) {
        const int q = NW * d + wave;
        if (d < XL) {
            const int row = q * (1024 / XROW) + lane / XCH;
            const int chunk = (lane % XCH) ^ wswz<XCH>(row);
            const int j = jb * BJ + chunk * 8;
            d_row[d] = row;
            d_chan[d] = j < a.Cg ? uint32_t((g * a.Cg + j) * 2) : kOob;
        } else {
            const int row = (q - XD) * (1024 / YROW) + lane / YCH;
            const int chunk = (lane % YCH) ^ wswz<YCH>(row);
            const int k = kb * kWBK + chunk * 8;
            d_row[d] = row;
            d_chan[d] = k < a.Kg ? uint32_t((g * a.Kg + k) * 2) : kOob;
        }
    }
    // Input gather state of each input slot, for the pixel m its lane loads in
    // the next issued stage: output row ho and column wo, and the byte offset
    // of input pixel (n, ho*s, wo*s).  It advances by 32 pixels per stage with
    // adds and compares only (no division in the loop).  The tap's input pixel
    // is that offset plus a per-block constant; it lies inside the image iff
    // ho and wo fall in the tap's valid ranges [ho_lo, ho_lo + ho_cnt) and
    // [wo_lo, wo_lo + wo_cnt).
    const uint32_t C2 = uint32_t(a.C) * 2u;
    int g_ho[XL], g_wo[XL];
    uint32_t g_pix[XL], g_cst[XL];
    int ho_lo = 0, wo_lo = 0;
    uint32_t ho_cnt = 0, wo_cnt = 0;
    uint32_t step_pix = 0, wrap_w = 0, wrap_h = 0;
    if constexpr (!PW) {
        const int s = a.stride;
        ho_lo = a.pad_h > r ? (a.pad_h - r + s - 1) / s : 0;
        wo_lo = a.pad_w > t ? (a.pad_w - t + s - 1) / s : 0;
        const int bh = a.H - 1 + a.pad_h - r, bw = a.W - 1 + a.pad_w - t;
        const int ho_hi = bh < 0 ? 0 : min(a.Ho, bh / s + 1);
        const int wo_hi = bw < 0 ? 0 : min(a.Wo, bw / s + 1);
        ho_cnt = uint32_t(max(0, ho_hi - ho_lo));
        wo_cnt = uint32_t(max(0, wo_hi - wo_lo));
        const uint32_t rowb = uint32_t(s) * uint32_t(a.W) * C2;   // one output row down
        const uint32_t colb = uint32_t(s) * C2;                   // one output column right
        step_pix = uint32_t(a.step_ho) * rowb + uint32_t(a.step_wo) * colb;
        wrap_w = rowb - uint32_t(a.Wo) * colb;
        wrap_h = uint32_t(a.H) * uint32_t(a.W) * C2 - uint32_t(a.Ho) * rowb;
        const uint32_t tap_b = uint32_t((r - a.pad_h) * a.W + (t - a.pad_w)) * C2;
#pragma unroll
        for (int d = 0; d < XL; ++d) {
            const int m = m_begin + d_row[d];
            const int n = fdiv(m, a.div_hw);
            const int rem = m - n * (a.Ho * a.Wo);
            const int ho = fdiv(rem, a.div_w);
            const int wo = rem - ho * a.Wo;
            g_ho[d] = ho;
            g_wo[d] = wo;
            g_pix[d] = uint32_t((n * a.H + ho * s) * a.W + wo * s) * C2;
            g_cst[d] = tap_b + d_chan[d];
        }
    }
    int g_m = m_begin;           // first pixel of the next issued stage
    // issue the loads of stage slot SL for pixels g_m .. g_m+31, then advance
    auto issue = [&](auto slot) {
        constexpr int SL = decltype(slot)::value;
#pragma unroll
        for (int d = 0; d < LPS; ++d) {
            const int m = g_m + d_row[d];
            unsigned char* dst = lds + SL * STAGE + (NW * d + wave) * 1024;
            if (d < XL) {
                uint32_t off = kOob;
                if constexpr (PW) {
                    if (m < m_end && d_chan[d] != kOob) off = uint32_t(m) * C2 + d_chan[d];
                } else {
                    const bool ok = m < m_end && d_chan[d] != kOob &&
                                    uint32_t(g_ho[d] - ho_lo) < ho_cnt &&
                                    uint32_t(g_wo[d] - wo_lo) < wo_cnt;
                    off = ok ? g_pix[d] + g_cst[d] : kOob;
                    g_wo[d] += a.step_wo;
                    g_ho[d] += a.step_ho;
                    g_pix[d] += step_pix;
                    if (g_wo[d] >= a.Wo) { g_wo[d] -= a.Wo; g_ho[d] += 1; g_pix[d] += wrap_w; }
                    while (g_ho[d] >= a.Ho) { g_ho[d] -= a.Ho; g_pix[d] += wrap_h; }
                }
                dma16(rx, dst, off, 0);
            } else {
                const uint32_t off = (m < m_end && d_chan[d] != kOob)
                                         ? uint32_t(m) * uint32_t(a.K * 2) + d_chan[d]
                                         : kOob;
                dma16(rdy, dst, off, 0);
            }
        }
        g_m += kWBM;
    };

    // ---- fragment read addresses (within a stage): lane (frow, fgrp), half h
    // of the 8 pixels fgrp*8.., reads pixel row fgrp*8 + 4h + frow/4, channels
    // tile*16 + 4*(frow%4) .. +3; the transpose hands it 4 pixels of channel
    // tile*16 + frow ----
    const int wj = wave % WAVES_J, wk = wave / WAVES_J;
    const uint32_t lds0 = lds_addr(lds);
    uint32_t xa[WJT][2], ya[WKT][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = fgrp * 8 + 4 * h + (frow >> 2);
#pragma unroll
        for (int jt = 0; jt < WJT; ++jt) {
            const int j = wj * 64 + jt * 16 + 4 * (frow & 3);
            xa[jt][h] = lds0 + row * XROW + (((j >> 3) ^ wswz<XCH>(row)) << 4) + (j & 7) * 2;
        }
#pragma unroll
        for (int kt = 0; kt < WKT; ++kt) {
            const int k = wk * (WKT * 16) + kt * 16 + 4 * (frow & 3);
            ya[kt][h] = lds0 + XBYTES + row * YROW + (((k >> 3) ^ wswz<YCH>(row)) << 4) + (k & 7) * 2;
        }
    }

    f32x4 acc[WJT][WKT];
#pragma unroll
    for (int i = 0; i < WJT; ++i)
#pragma unroll
        for (int j = 0; j < WKT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // multiply the stage in slot SL
    auto compute = [&](auto slot) {
        constexpr int SL = decltype(slot)::value;
        i32x2 fx[WJT][2], fy[WKT][2];
#pragma unroll
        for (int jt = 0; jt < WJT; ++jt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                             : "=v"(fx[jt][h]) : "v"(xa[jt][h]), "i"(SL * STAGE));
#pragma unroll
        for (int kt = 0; kt < WKT; ++kt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                             : "=v"(fy[kt][h]) : "v"(ya[kt][h]), "i"(SL * STAGE));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int jt = 0; jt < WJT; ++jt) {
            asm volatile("" : "+v"(fx[jt][0]), "+v"(fx[jt][1]));
            const i32x4 av = {fx[jt][0][0], fx[jt][0][1], fx[jt][1][0], fx[jt][1][1]};
#pragma unroll
            for (int kt = 0; kt < WKT; ++kt) {
                if (jt == 0) asm volatile("" : "+v"(fy[kt][0]), "+v"(fy[kt][1]));
                const i32x4 bv = {fy[kt][0][0], fy[kt][0][1], fy[kt][1][0], fy[kt][1][1]};
                acc[jt][kt] = mfma16x16x32<T>(av, bv, acc[jt][kt]);
            }
        }
    };

    // ---- ring: stages 0..2 in flight before the first multiply ----
    sfor<kWStages - 1>([&](auto sc) { issue(sc); });
    for (int s0 = 0; s0 < nsteps; s0 += kWStages) {
        sfor<kWStages>([&](auto sc) {
            constexpr int SL = decltype(sc)::value;
            const int s = s0 + SL;
            if (s < nsteps) {
                wait_vm<(kWStages - 2) * LPS>();
                __builtin_amdgcn_s_barrier();
                // the slot freed by the previous stage takes stage s + 3
                issue(IC<(SL + kWStages - 1) % kWStages>{});
                compute(IC<SL>{});
            }
        });
    }
    wait_vm<0>();   // no DMA may still be writing LDS when the block retires

    // ---- fp32 partials: lane holds j rows 4*fgrp..+3 of k column frow ----
    float* wsp = a.ws + int64_t(split) * a.split_elems;
#pragma unroll
    for (int kt = 0; kt < WKT; ++kt) {
        const int k = kb * kWBK + wk * (WKT * 16) + kt * 16 + frow;
        if (k >= a.Kg) continue;
        float* rowp = wsp + (int64_t(g * a.Kg + k) * RS + tap) * a.Cg;
#pragma unroll
        for (int jt = 0; jt < WJT; ++jt) {
            const int j = jb * BJ + wj * 64 + jt * 16 + 4 * fgrp;
            if (j < a.Cg) *reinterpret_cast<f32x4*>(rowp + j) = acc[jt][kt];
        }
    }
}

// dw[i] = round(sum over splits of ws[s][i]), four elements per lane group.
// L lanes (a power of two <= 16, consecutive in one wave) share an element:
// lane q adds the contiguous split range [q*S/L, (q+1)*S/L) in ascending
// order, eight loads in flight, and the first lane of the group then adds the
// L range sums in ascending q.  A fixed order, so the result is reproducible;
// with L = 1 it is the plain ascending sum.
template <typename T>
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ ws,
                                                           unsigned short* __restrict__ dw,
                                                           int64_t total4, int64_t stride4,
                                                           int splits, int lshift) {
    const int L = 1 << lshift;
    const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t i = gid >> lshift;
    const int q = int(gid & (L - 1));
    const bool valid = i < total4;
    const int s0 = int(int64_t(q) * splits >> lshift), s1 = int(int64_t(q + 1) * splits >> lshift);
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    if (valid && s0 < s1) {
        const f32x4* src = reinterpret_cast<const f32x4*>(ws) + i;
        s = src[int64_t(s0) * stride4];
        for (int sp0 = s0 + 1; sp0 < s1; sp0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (sp0 + j < s1) v[j] = src[int64_t(sp0 + j) * stride4];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (sp0 + j < s1) {
                    s[0] += v[j][0]; s[1] += v[j][1]; s[2] += v[j][2]; s[3] += v[j][3];
                }
        }
    }
    // every lane of the wave takes part in the shuffles (no early exit above)
    const int lane = int(threadIdx.x & 63), base = lane & ~(L - 1);
    f32x4 t = s;
    for (int k = 1; k < L; ++k) {
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = __shfl(s[c], base + k, 64);
        t[0] += v[0]; t[1] += v[1]; t[2] += v[2]; t[3] += v[3];
    }
    if (valid && q == 0) {
        i32x2 o = {int(pack2<T>(t[0], t[1])), int(pack2<T>(t[2], t[3]))};
        *(reinterpret_cast<i32x2*>(dw) + i) = o;
    }
}

// One weight element per lane, pixels in (n, ho, wo) order, fp32 accumulation.
template <typename T>
__global__ __launch_bounds__(256) void wgrad_generic_kernel(
    const unsigned short* __restrict__ x, const unsigned short* __restrict__ dy,
    unsigned short* __restrict__ dw, int64_t total, int N, int H, int W, int C, int K, int R, int S,
    int stride, int pad_h, int pad_w, int Ho, int Wo, int Cg, int Kg) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int j = int(i % Cg);
    int64_t q = i / Cg;
    const int t = int(q % S);
    q /= S;
    const int r = int(q % R);
    const int k = int(q / R);
    const int g = k / Kg;
    float acc = 0.f;
    for (int n = 0; n < N; ++n)
        for (int ho = 0; ho < Ho; ++ho) {
            const int h = ho * stride - pad_h + r;
            if (h < 0 || h >= H) continue;
            for (int wo = 0; wo < Wo; ++wo) {
                const int w = wo * stride - pad_w + t;
                if (w < 0 || w >= W) continue;
                acc += to_f32<T>(dy[((int64_t(n) * Ho + ho) * Wo + wo) * K + k]) *
                       to_f32<T>(x[((int64_t(n) * H + h) * W + w) * C + g * Cg + j]);
            }
        }
    dw[i] = pack1<T>(acc);
}

int wg_bj(const Prob& p) { return p.cg >= 128 ? 128 : 64; }
// waves per block: 8 (256 output channels) for wide groups on both sides
int wg_nw(const Prob& p) { return (wg_bj(p) == 128 && p.kg > 128) ? 8 : 4; }

int64_t wg_tiles(const Prob& p) {
    const int bj = wg_bj(p), kb = wg_kb(wg_nw(p));
    return int64_t(p.groups) * ((p.kg + kb - 1) / kb) * p.r * p.s * ((p.cg + bj - 1) / bj);
}

}  // namespace

std::string wgrad_splitk_reason(const Prob& p, bool pointwise) {
    if (pointwise && !(p.r == 1 && p.s == 1 && p.stride == 1 && p.pad_h == 0 && p.pad_w == 0))
        return "pointwise wgrad needs a 1x1 filter, stride 1 and no padding";
    if (p.cg % 8 != 0 || p.kg % 8 != 0)
        return "needs C/groups and K/groups multiples of 8 (16-byte rows)";
    if (p.cg < 16 || p.kg < 16)
        return "needs at least 16 channels per group on each side (MFMA tile)";
    if (p.ho * p.wo > (int64_t(1) << 30) || p.h * p.w > (int64_t(1) << 30))
        return "feature map too large for the kernel's 32-bit pixel indices";
    return "";
}

int wgrad_splits(const Prob& p, int tune) {
    if (tune > 0) return int(std::min<int64_t>(tune, p.n * p.ho * p.wo));
    const int64_t tiles = wg_tiles(p);
    const int64_t P = p.n * p.ho * p.wo;
    if (wg_nw(p) == 8) {
        // 8-wave blocks: at most one per compute unit (a second block on a CU
        // halves both; 3x3 256-channel workload: 14 splits = 252 blocks 51.0
        // us, 16 splits = 288 blocks 74.8 us), every split at least 8 stages
        int64_t s = std::max<int64_t>(1, kNumCUs / tiles);
        return int(std::max<int64_t>(1, std::min<int64_t>(s, P / (8 * kWBM))));
    }
    // One block per compute unit, every split at least 8 stages deep.  More
    // splits shorten the blocks but each adds a full fp32 partial of dW to
    // the workspace traffic (written here, read by the reduce).
    int64_t s = std::max<int64_t>(1, (kNumCUs + tiles - 1) / tiles);
    s = std::min<int64_t>(s, std::max<int64_t>(1, P / (8 * kWBM)));
    // a multiple of 8 blocks lets the XCD remap deal contiguous runs
    while ((s * tiles) % 8 != 0 && (s + 1) <= P / kWBM && s < 4 * (2 * kNumCUs)) ++s;
    return int(s);
}

int64_t wgrad_split_elems(const Prob& p) { return p.k * p.r * p.s * p.cg; }

int launch_wgrad_splitk(const Prob& p, const Plan& pl, const void* x, const void* dy, float* ws,
                        int splits, hipStream_t st) {
    WgArgs a;
    a.x = x; a.dy = dy; a.ws = ws;
    a.x_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg);
    a.P = int(p.n * p.ho * p.wo);
    const int bj = wg_bj(p);
    const int nw = wg_nw(p);
    a.kblocks = int((p.kg + wg_kb(nw) - 1) / wg_kb(nw));
    a.jblocks = int((p.cg + bj - 1) / bj);
    a.tiles = int(wg_tiles(p));
    a.splits = splits;
    a.div_hw = make_fastdiv(uint32_t(p.ho * p.wo));
    a.div_w = make_fastdiv(uint32_t(p.wo));
    a.step_ho = int(kWBM / p.wo);
    a.step_wo = int(kWBM % p.wo);
    a.split_elems = wgrad_split_elems(p);
    const int64_t blocks = int64_t(a.tiles) * splits;
    if (blocks > (int64_t(1) << 31) - 1) return CNHWC_UNSUPPORTED;
    a.remap = 1;
    const bool pw = pl.variant == CNHWC_VAR_WGRAD_POINTWISE;
    const bool bf = p.dtype == CNHWC_BF16;
#define CNHWC_WG(T, BJ, PW, NW) hipLaunchKernelGGL((wgrad_splitk_kernel<T, BJ, PW, NW>), dim3(unsigned(blocks)), \
                                                   dim3(NW * 64), 0, st, a)
    if (bj == 128 && nw == 8) {
        if (pw) { if (bf) CNHWC_WG(BF16, 128, true, 8); else CNHWC_WG(F16, 128, true, 8); }
        else { if (bf) CNHWC_WG(BF16, 128, false, 8); else CNHWC_WG(F16, 128, false, 8); }
    } else if (bj == 128) {
        if (pw) { if (bf) CNHWC_WG(BF16, 128, true, 4); else CNHWC_WG(F16, 128, true, 4); }
        else { if (bf) CNHWC_WG(BF16, 128, false, 4); else CNHWC_WG(F16, 128, false, 4); }
    } else {
        if (pw) { if (bf) CNHWC_WG(BF16, 64, true, 4); else CNHWC_WG(F16, 64, true, 4); }
        else { if (bf) CNHWC_WG(BF16, 64, false, 4); else CNHWC_WG(F16, 64, false, 4); }
    }
#undef CNHWC_WG
    return CNHWC_OK;
}

int launch_wgrad_reduce(const Prob& p, int splits, const float* ws, void* dw, hipStream_t st) {
    const int64_t total4 = wgrad_split_elems(p) / 4;
    // lanes per element: enough that each adds at most 8 splits, at most 16
    int lshift = 0;
    while (lshift < 4 && (int64_t(splits) + (int64_t(1) << lshift) - 1) >> lshift > 8) ++lshift;
    const int64_t blocks = ((total4 << lshift) + 255) / 256;
    if (blocks > (int64_t(1) << 31) - 1) return CNHWC_UNSUPPORTED;
    auto* out = static_cast<unsigned short*>(dw);
    if (p.dtype == CNHWC_BF16)
        hipLaunchKernelGGL(wgrad_reduce_kernel<BF16>, dim3(unsigned(blocks)), dim3(256), 0, st, ws,
                           out, total4, total4, splits, lshift);
    else
        hipLaunchKernelGGL(wgrad_reduce_kernel<F16>, dim3(unsigned(blocks)), dim3(256), 0, st, ws,
                           out, total4, total4, splits, lshift);
    return CNHWC_OK;
}

int launch_wgrad_generic(const Prob& p, const void* x, const void* dy, void* dw, hipStream_t st) {
    const int64_t total = wgrad_split_elems(p);
    const unsigned blocks = unsigned((total + 255) / 256);
    auto* xs = static_cast<const unsigned short*>(x);
    auto* ys = static_cast<const unsigned short*>(dy);
    auto* out = static_cast<unsigned short*>(dw);
#define CNHWC_WGG(T) hipLaunchKernelGGL(wgrad_generic_kernel<T>, dim3(blocks), dim3(256), 0, st, xs, ys, \
                                        out, total, int(p.n), int(p.h), int(p.w), int(p.c), int(p.k),     \
                                        int(p.r), int(p.s), p.stride, p.pad_h, p.pad_w, int(p.ho),        \
                                        int(p.wo), int(p.cg), int(p.kg))
    if (p.dtype == CNHWC_BF16) CNHWC_WGG(BF16);
    else CNHWC_WGG(F16);
#undef CNHWC_WGG
    return CNHWC_OK;
}

}  // namespace cnhwc
