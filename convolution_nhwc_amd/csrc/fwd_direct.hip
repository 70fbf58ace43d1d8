// Direct forward convolution on the gfx950 matrix cores with the input tile and
// its halo staged in LDS ("feat(rocke): split-C and grouped LDS-halo direct
// conv fwd kernels"):
//
//  * fwd_direct: a block owns an output tile of NB images x TH rows x TW
//    columns (<= 128 pixels, the MFMA M side) and BN = 64 output channels.
//    Per 64-channel chunk the input window ((TH-1)*s+R) x ((TW-1)*s+S) of those
//    channels is loaded into LDS once and every filter tap reads a shifted
//    window of it; the weight slice of the tap streams through LDS.  Both
//    operands are channel-contiguous, which is what the MFMA reduction wants,
//    so nothing is transposed.
//  * split_c: the same kernel with the channel loop split across blocks
//    (grid axis = split index); each split writes its fp32 partial tile to a
//    workspace [split][pixel][k] and a second pass, split_reduce, sums the
//    splits in ascending order and rounds once.  This fills the GPU when the
//    output has too few tiles (small maps, deep channels).
//  * grouped merge: with few channels per group, G_m = 32/Cg groups are merged
//    into one MFMA problem -- 32 input channels x G_m*Kg output channels --
//    whose per-tap weight tile is block-diagonal (zero off the group blocks),
//    so one MFMA covers several groups instead of leaving most of the tile idle.
//
// Block ids are remapped so that the blocks sharing one weight slice run on the
// same XCD (blocks are dealt to the 8 XCDs round-robin; each XCD has its own
// L2).  Out-of-image pixels and out-of-range channels read zero through the
// buffer descriptors' range check.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>

namespace cnhwc {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;          // output pixels per block (MFMA M)
constexpr int kBN = 64;           // output channels per block (direct)
constexpr int kBKc = 64;          // input channels per LDS stage (direct)
constexpr int kHaloMax = 336;     // halo pixels per stage (42 KiB at 128 B/pixel)
constexpr int kHaloSlots = (kHaloMax * 8 + kThreads - 1) / kThreads;

struct Geo {
    int NB, TH, TW;   // tile: images x rows x columns
    int IH, IW;       // halo rows / columns
    int ptiles_h, ptiles_w, ptiles_n;
};

struct FwdArgs {
    const void* x;
    const void* w;
    void* y;          // output (unsplit) or fp32 workspace (split)
    uint32_t x_bytes, w_bytes, y_bytes;
    int N, H, W, C, K, R, S, stride, pad_h, pad_w, Ho, Wo, Cg, Kg, G;
    Geo geo;
    int ntiles;       // output-channel tiles per group
    int splits, csplit;   // channel splits and channels per split
    int nblocks;
    int remap;
    int halo_bytes;   // LDS bytes of one halo stage
};

__device__ inline uint32_t swz(int row, int chunk) { return uint32_t((chunk ^ (row & 7)) * 16); }

// Decode a tile index into its first image / output row / output column.
__device__ inline void tile_origin(const Geo& g, int pt, int& n0, int& ho0, int& wo0) {
    const int tw = pt % g.ptiles_w;
    const int rest = pt / g.ptiles_w;
    const int th = rest % g.ptiles_h;
    n0 = (rest / g.ptiles_h) * g.NB;
    ho0 = th * g.TH;
    wo0 = tw * g.TW;
}

template <typename T, bool SPLIT>
__global__ __launch_bounds__(kThreads) void fwd_direct_kernel(const FwdArgs a) {
    constexpr int B_BYTES = kBN * 128;
    constexpr int WM = kBM / 2, WN = kBN / 2, FM = WM / 16, FN = WN / 16;
    // dynamic LDS: [halo 0][halo 1][weights 0][weights 1]; halo = a.halo_bytes
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int HALO_BYTES = a.halo_bytes;
    unsigned char* const wbase = lds + 2 * HALO_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Geo& geo = a.geo;

    int bid = blockIdx.x;
    if (a.remap) bid = (bid & 7) * (a.nblocks >> 3) + (bid >> 3);
    const int ptiles = geo.ptiles_n * geo.ptiles_h * geo.ptiles_w;
    const int pt = bid % ptiles;
    int rest = bid / ptiles;
    const int nt = rest % a.ntiles;
    rest /= a.ntiles;
    const int g = rest % a.G;
    const int sp = rest / a.G;
    int n0, ho0, wo0;
    tile_origin(geo, pt, n0, ho0, wo0);
    const int k0 = nt * kBN;                 // within the group
    const int c_lo = sp * a.csplit;          // within the group
    const int c_hi = min(a.Cg, c_lo + a.csplit);
    const int s = a.stride;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);

    // halo slots of this thread: chunk (tid & 7) of halo pixels tid/8 + 32 j
    const int hchunk = tid & 7;
    const int hpix = geo.NB * geo.IH * geo.IW;
    int hoff[kHaloSlots];
#pragma unroll
    for (int j = 0; j < kHaloSlots; ++j) {
        const int hp = (tid >> 3) + j * (kThreads / 8);
        hoff[j] = -1;
        if (hp < hpix) {
            const int per = geo.IH * geo.IW;
            const int nb = hp / per;
            const int rem = hp - nb * per;
            const int ih = rem / geo.IW, iw = rem - (rem / geo.IW) * geo.IW;
            const int n = n0 + nb;
            const int h = ho0 * s - a.pad_h + ih, w = wo0 * s - a.pad_w + iw;
            if (n < a.N && h >= 0 && h < a.H && w >= 0 && w < a.W)
                hoff[j] = ((n * a.H + h) * a.W + w) * a.C + g * a.Cg;
        }
    }
    // weight rows of this thread: chunk (tid & 7) of rows tid/8 + 32 j
    const int taps = a.R * a.S;
    const int cchunks = (c_hi - c_lo + kBKc - 1) / kBKc;
    const int steps = cchunks * taps;

    i32x4 rh[kHaloSlots];
    i32x4 rb[2];

    auto load_halo = [&](int cc) {
        const int c = c_lo + cc * kBKc + hchunk * 8;
#pragma unroll
        for (int j = 0; j < kHaloSlots; ++j) {
            const uint32_t off = (hoff[j] >= 0 && c < c_hi) ? uint32_t(hoff[j] + c) * 2u : kOob;
            rh[j] = buf_load16(rx, off);
        }
    };
    auto load_w = [&](int cc, int tap) {
        const int c = c_lo + cc * kBKc + hchunk * 8;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kr = (tid >> 3) + j * 32;
            const int k = k0 + kr;
            uint32_t off = kOob;
            if (k < a.Kg && c < c_hi)
                off = uint32_t(((g * a.Kg + k) * taps + tap) * a.Cg + c) * 2u;
            rb[j] = buf_load16(rw, off);
        }
    };
    auto store_halo = [&](int buf) {
        unsigned char* hs = lds + buf * HALO_BYTES;
#pragma unroll
        for (int j = 0; j < kHaloSlots; ++j) {
            const int hp = (tid >> 3) + j * (kThreads / 8);
            if (hp < hpix) *reinterpret_cast<i32x4*>(hs + hp * 128 + swz(hp, hchunk)) = rh[j];
        }
    };
    auto store_w = [&](int buf) {
        unsigned char* bs = wbase + buf * B_BYTES;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kr = (tid >> 3) + j * 32;
            *reinterpret_cast<i32x4*>(bs + kr * 128 + swz(kr, hchunk)) = rb[j];
        }
    };

    // fragment rows: output pixel -> base halo index (tap 0)
    const int wm = wave >> 1, wn = wave & 1;
    const int frow = lane & 15, fgrp = lane >> 4;
    const int tile_pix = geo.NB * geo.TH * geo.TW;
    int fbase[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        int m = wm * WM + i * 16 + frow;
        if (m >= tile_pix) m = 0;
        const int per = geo.TH * geo.TW;
        const int nb = m / per;
        const int rem = m - nb * per;
        const int th = rem / geo.TW, tw = rem - (rem / geo.TW) * geo.TW;
        fbase[i] = nb * geo.IH * geo.IW + th * s * geo.IW + tw * s;
    }

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, int tap) {
        const unsigned char* hs = lds + buf * HALO_BYTES;
        const unsigned char* bs = wbase + buf * B_BYTES;
        const int r = tap / a.S, t = tap - (tap / a.S) * a.S;
        const int toff = r * geo.IW + t;
#pragma unroll
        for (int ks = 0; ks < kBKc / 32; ++ks) {
            const int chunk = ks * 4 + fgrp;
            i32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int hp = fbase[i] + toff;
                fa[i] = *reinterpret_cast<const i32x4*>(hs + hp * 128 + swz(hp, chunk));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int kr = wn * WN + j * 16 + frow;
                fb[j] = *reinterpret_cast<const i32x4*>(bs + kr * 128 + swz(kr, chunk));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<T>(fb[j], fa[i], acc[i][j]);
        }
    };

    // The halo buffer of a stage is only rewritten at a chunk boundary; the
    // halo in buffer b stays valid for all taps that use buffer b... so the
    // halo is kept per chunk parity and the weight slice per step parity.
    if (steps > 0) {
        load_halo(0);
        load_w(0, 0);
        store_halo(0);
        store_w(0);
        __syncthreads();
#pragma unroll 1
        for (int st = 0; st < steps; ++st) {
            const int cc = st / taps, tap = st - cc * taps;
            const bool more = st + 1 < steps;
            const bool new_chunk = more && tap + 1 == taps;
            if (more) {
                if (new_chunk) load_halo(cc + 1);
                load_w(tap + 1 == taps ? cc + 1 : cc, tap + 1 == taps ? 0 : tap + 1);
            }
            // halo of chunk cc sits in buffer (cc & 1); weights of step st in (st & 1)
            {
                const unsigned char* hs = lds + (cc & 1) * HALO_BYTES;
                const unsigned char* bs = wbase + (st & 1) * B_BYTES;
                const int r = tap / a.S, t = tap - (tap / a.S) * a.S;
                const int toff = r * geo.IW + t;
#pragma unroll
                for (int ks = 0; ks < kBKc / 32; ++ks) {
                    const int chunk = ks * 4 + fgrp;
                    i32x4 fa[FM], fb[FN];
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const int hp = fbase[i] + toff;
                        fa[i] = *reinterpret_cast<const i32x4*>(hs + hp * 128 + swz(hp, chunk));
                    }
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int kr = wn * WN + j * 16 + frow;
                        fb[j] = *reinterpret_cast<const i32x4*>(bs + kr * 128 + swz(kr, chunk));
                    }
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = mfma16x16x32<T>(fb[j], fa[i], acc[i][j]);
                }
            }
            if (more) {
                if (new_chunk) store_halo((cc + 1) & 1);
                store_w((st + 1) & 1);
            }
            __syncthreads();
        }
    }
    (void)compute;

    // ---- epilogue through LDS: rows = tile pixels, columns = BN channels ----
    constexpr int ESZ = SPLIT ? 4 : 2;
    constexpr int C_STRIDE = kBN * ESZ + 16;
    // the launcher sizes LDS to at least kBM * C_STRIDE for the epilogue tile
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wm * WM + i * 16 + frow;
            const int col = wn * WN + j * 16 + fgrp * 4;
            if constexpr (SPLIT) {
                *reinterpret_cast<f32x4*>(lds + row * C_STRIDE + col * 4) = acc[i][j];
            } else {
                i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                           int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
                *reinterpret_cast<i32x2*>(lds + row * C_STRIDE + col * 2) = v;
            }
        }
    __syncthreads();
    constexpr int CPR = kBN * ESZ / 16;
    const int64_t mtotal = int64_t(a.N) * a.Ho * a.Wo;
    for (int q = tid; q < kBM * CPR; q += kThreads) {
        const int row = q / CPR, cc = q % CPR;
        if (row >= tile_pix) continue;
        const int per = geo.TH * geo.TW;
        const int nb = row / per;
        const int rem = row - nb * per;
        const int th = rem / geo.TW, tw = rem - (rem / geo.TW) * geo.TW;
        const int n = n0 + nb, ho = ho0 + th, wo = wo0 + tw;
        if (n >= a.N || ho >= a.Ho || wo >= a.Wo) continue;
        const int kl = k0 + cc * (16 / ESZ);
        if (kl >= a.Kg) continue;
        const int pix = (n * a.Ho + ho) * a.Wo + wo;
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + row * C_STRIDE + cc * 16);
        if constexpr (SPLIT) {
            const int64_t e = (int64_t(sp) * mtotal + pix) * a.K + g * a.Kg + kl;
            buf_store16(v, ry, uint32_t(e) * 4u);
        } else {
            buf_store16(v, ry, uint32_t(pix * a.K + g * a.Kg + kl) * 2u);
        }
    }
}

// y[i] = round(sum over splits, ascending, of ws[split][i]), 4 elements a lane.
template <typename T>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ ws,
                                                           unsigned short* __restrict__ y,
                                                           int64_t total4, int64_t stride4,
                                                           int splits) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total4;
         i += int64_t(gridDim.x) * blockDim.x) {
        f32x4 s = reinterpret_cast<const f32x4*>(ws)[i];
        // sixteen splits' loads are in flight at once (one memory round trip
        // for up to 17 splits); the adds stay in ascending split order
        constexpr int kBatch = 16;
        for (int sp0 = 1; sp0 < splits; sp0 += kBatch) {
            f32x4 v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (sp0 + j < splits) v[j] = reinterpret_cast<const f32x4*>(ws)[i + (sp0 + j) * stride4];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (sp0 + j < splits) {
                    s[0] += v[j][0]; s[1] += v[j][1]; s[2] += v[j][2]; s[3] += v[j][3];
                }
        }
        i32x2 o = {int(pack2<T>(s[0], s[1])), int(pack2<T>(s[2], s[3]))};
        __builtin_nontemporal_store(o, reinterpret_cast<i32x2*>(y) + i);
    }
}

// ---- grouped merge ----------------------------------------------------------
constexpr int kGBK = 32;          // merged input channels (MFMA reduction)
constexpr int kGHaloMax = 336;    // halo pixels (64 B each)
constexpr int kGHaloSlots = (kGHaloMax * 4 + kThreads - 1) / kThreads;
constexpr int kMaxTaps = 25;

struct GrpArgs {
    const void* x;
    const void* w;
    void* y;
    uint32_t x_bytes, w_bytes, y_bytes;
    int N, H, W, C, K, R, S, stride, pad_h, pad_w, Ho, Wo, Cg, Kg, G;
    int gm;           // groups merged per block
    int bn;           // gm * Kg output channels per block (multiple of 16, <= 64)
    int gsets;        // G / gm
    Geo geo;
    int nblocks, remap;
    int halo_bytes;   // LDS bytes of the halo (start of the weight taps)
    FastDiv fd_img, fd_iw, fd_per, fd_tw;   // division by IH*IW, IW, TH*TW, TW
};

template <typename T, int BN>
__global__ __launch_bounds__(kThreads) void fwd_grouped_kernel(const GrpArgs a) {
    constexpr int W_TAP = BN * 64;              // one tap: BN rows x 32 channels
    constexpr int FM = kBM / 16 / 4;            // 2 row blocks per wave (waves split M)
    constexpr int FN = BN / 16;
    // dynamic LDS: the halo (64 B a pixel) then the block-diagonal taps
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char* hs = lds;
    unsigned char* ws = lds + a.halo_bytes;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Geo& geo = a.geo;
    int bid = blockIdx.x;
    if (a.remap) bid = (bid & 7) * (a.nblocks >> 3) + (bid >> 3);
    const int ptiles = geo.ptiles_n * geo.ptiles_h * geo.ptiles_w;
    const int pt = bid % ptiles;
    const int gs = bid / ptiles;
    int n0, ho0, wo0;
    tile_origin(geo, pt, n0, ho0, wo0);
    const int s = a.stride;
    const int taps = a.R * a.S;
    const int cbase = gs * a.gm * a.Cg;         // first input channel of the set
    const int kbase = gs * a.bn;                // first output channel of the set

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);

    // halo: 4 chunks of 8 channels per pixel, loaded straight into LDS (one
    // 16-pixel load per wave instruction; the chunk swizzle is applied on the
    // source side: lane -> (pixel, physical chunk), reading logical chunk
    // physical ^ (pixel & 3))
    const int hpix = geo.NB * geo.IH * geo.IW;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    for (int q0 = wv * 16; q0 < hpix; q0 += (kThreads / 64) * 16) {
        const int hp = q0 + (lane >> 2);
        const int hchunk = (lane & 3) ^ (hp & 3);
        const int nb = fdiv(hp, a.fd_img);
        const int rem = hp - nb * (geo.IH * geo.IW);
        const int ih = fdiv(rem, a.fd_iw), iw = rem - ih * geo.IW;
        const int n = n0 + nb;
        const int h = ho0 * s - a.pad_h + ih, w = wo0 * s - a.pad_w + iw;
        uint32_t off = kOob;
        if (hp < hpix && n < a.N && h >= 0 && h < a.H && w >= 0 && w < a.W)
            off = uint32_t(((n * a.H + h) * a.W + w) * a.C + cbase + hchunk * 8) * 2u;
        dma16(rx, hs + q0 * 64, off, 0);
    }
    // block-diagonal weights: row kk (output channel of the set) has the Cg
    // weights of its group at columns (kk / Kg) * Cg .. +Cg, zeros elsewhere.
    // Staged per 16-byte LDS chunk (8 merged channels of one row and tap).
    const int nchunks = taps * BN * 4;
    if (a.Cg % 8 == 0) {
        // every chunk lies inside one group's channel block or is zero (an
        // out-of-range load writes zeros): async loads, 16 rows per instruction
        for (int e0 = wv * 64; e0 < nchunks; e0 += kThreads) {
            const int e = e0 + lane;
            const int row = (e >> 2) % BN;
            const int tap = (e >> 2) / BN;
            const int c8 = (e & 3) ^ (row & 3);   // logical chunk held by this physical slot
            const int gl = row / a.Kg;
            const int k = kbase + row;
            uint32_t off = kOob;
            if (row < a.bn && (c8 * 8) / a.Cg == gl)
                off = uint32_t((k * taps + tap) * a.Cg + c8 * 8 - gl * a.Cg) * 2u;
            dma16(rw, ws + (e0 >> 2) * 64, off, 0);
        }
    } else {
    for (int e = tid; e < nchunks; e += kThreads) {
        const int c8 = e & 3;
        const int row = (e >> 2) % BN;
        const int tap = (e >> 2) / BN;
        const int gl = row / a.Kg;              // group of this output channel within the set
        const int k = kbase + row;
        i32x4 v = {0, 0, 0, 0};
        {
            // several groups share the chunk: element by element
            uint32_t h[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int col = c8 * 8 + q;
                h[q] = (row < a.bn && col / a.Cg == gl)
                           ? uint32_t(buf_load2(rw, uint32_t((k * taps + tap) * a.Cg + col - gl * a.Cg) * 2u))
                           : 0u;
            }
            v = i32x4{int(h[0] | (h[1] << 16)), int(h[2] | (h[3] << 16)), int(h[4] | (h[5] << 16)),
                      int(h[6] | (h[7] << 16))};
        }
        *reinterpret_cast<i32x4*>(ws + tap * W_TAP + row * 64 + ((c8 ^ (row & 3)) * 16)) = v;
    }
    }
    wait_vm<0>();
    __syncthreads();

    const int frow = lane & 15, fgrp = lane >> 4;
    const int tile_pix = geo.NB * geo.TH * geo.TW;
    int fbase[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        int m = wave * (kBM / 4) + i * 16 + frow;
        if (m >= tile_pix) m = 0;
        const int per = geo.TH * geo.TW;
        const int nb = m / per;
        const int rem = m - nb * per;
        const int th = rem / geo.TW, tw = rem - (rem / geo.TW) * geo.TW;
        fbase[i] = nb * geo.IH * geo.IW + th * s * geo.IW + tw * s;
    }
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int tap = 0; tap < taps; ++tap) {
        const int r = tap / a.S, t = tap - (tap / a.S) * a.S;
        const int toff = r * geo.IW + t;
        i32x4 fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int hp = fbase[i] + toff;
            fa[i] = *reinterpret_cast<const i32x4*>(hs + hp * 64 + ((fgrp ^ (hp & 3)) * 16));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = j * 16 + frow;
            fb[j] = *reinterpret_cast<const i32x4*>(ws + tap * W_TAP + row * 64 + ((fgrp ^ (row & 3)) * 16));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<T>(fb[j], fa[i], acc[i][j]);
    }
    __syncthreads();
    // epilogue: tile [128 pixels][BN] of 16-bit outputs staged in LDS
    constexpr int C_STRIDE = BN * 2 + 16;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wave * (kBM / 4) + i * 16 + frow;
            const int col = j * 16 + fgrp * 4;
            i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                       int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
            *reinterpret_cast<i32x2*>(lds + row * C_STRIDE + col * 2) = v;
        }
    __syncthreads();
    constexpr int CPR = BN / 8;
    for (int q = tid; q < kBM * CPR; q += kThreads) {
        const int row = q / CPR, cc = q % CPR;
        if (row >= tile_pix || cc * 8 >= a.bn) continue;
        const int per = geo.TH * geo.TW;
        const int nb = fdiv(row, a.fd_per);
        const int rem = row - nb * per;
        const int th = fdiv(rem, a.fd_tw), tw = rem - th * geo.TW;
        const int n = n0 + nb, ho = ho0 + th, wo = wo0 + tw;
        if (n >= a.N || ho >= a.Ho || wo >= a.Wo) continue;
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + row * C_STRIDE + cc * 16);
        buf_store16(v, ry, uint32_t(((n * a.Ho + ho) * a.Wo + wo) * a.K + kbase + cc * 8) * 2u);
    }
}

// ---- grouped merge, whole-pixel-row variant ---------------------------------
// Same MFMA problem per group set as fwd_grouped_kernel (32 merged input
// channels x G_m*Kg outputs, block-diagonal weights), organised around HBM
// access: a block owns TH x TW output pixels of one image for ALL channels,
// so its input halo arrives as whole pixel rows (C*2 contiguous bytes per
// pixel, 1 KiB per load instruction) instead of 64-byte slices, and its
// output leaves as whole rows.  Eight waves; wave w computes group sets w,
// w+8, ...; each holds its set's block-diagonal weight fragments in registers
// (loaded straight from the filter as stored: lanes whose 8 merged channels
// belong to another group read out of range, i.e. zeros) and reads the
// input fragments from the halo (16-byte chunks XOR-ed by pixel & 15, or & 7
// for rows of fewer chunks, applied to the source addresses).  Results are rounded into an output tile in LDS
// and stored as contiguous rows at the end.
constexpr int kGrThreads = 512;

struct GrowArgs {
    const void* x;
    const void* w;
    void* y;
    uint32_t x_bytes, w_bytes, y_bytes;
    int N, H, W, C, K, stride, pad_h, pad_w, Ho, Wo, Cg, Kg;
    int bn, gsets;                // outputs per group set, group sets
    int TH, TW, IH, IW;           // output tile, input halo
    int ptiles_h, ptiles_w;       // tiles per image
    int halo_bytes;               // LDS of the halo (whole 1 KiB loads)
    int hmask, omask;             // chunk swizzle masks: 15 when a row has 16k chunks, else 7
    FastDiv fd_cpr, fd_iw, fd_tw, fd_kc;   // division by C/8, IW, TW, K/8
    int dg_lds;                   // DG: stage each wave's filter slice through LDS (one set a wave)
    FastDiv fd_kg, fd_cg;         // division by Kg, Cg
};

// DG (1: filter gathered per fragment, 2: staged through LDS; 0: forward):
// the same correlation run for grouped dgrad at stride 1 (x = dY, y = dX,
// padding R-1-pad): element (o, tap, i) of the correlation's filter is then
// W[g*Cg + i][R-1-r][S-1-t][o - g*Kg] of the stored filter (Cg, Kg here are the
// correlation's input and output channels per group).
template <typename T, int BN, int R, int S, int DG>
__global__ __launch_bounds__(kGrThreads, 1) void fwd_grouped_rows_kernel(const GrowArgs a) {
    constexpr int TAPS = R * S, FM = kBM / 16, FN = BN / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char* hs = lds;                       // halo [pixel][C]
    unsigned char* os = lds + a.halo_bytes;        // output tile [pixel][K]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per_img = a.ptiles_h * a.ptiles_w;
    // each XCD (blockIdx % 8) takes a contiguous run of tiles: neighbouring
    // tiles of an image, which read the same halo rows, share its L2
    int bid = blockIdx.x;
    {
        const int q = int(gridDim.x >> 3), rr = int(gridDim.x & 7), x = bid & 7;
        bid = x * q + min(x, rr) + (bid >> 3);
    }
    const int n = bid / per_img;
    const int pt = bid - n * per_img;
    const int ho0 = (pt / a.ptiles_w) * a.TH, wo0 = (pt % a.ptiles_w) * a.TW;
    const int s = a.stride;
    const int cpr = a.C / 8;                       // 16-byte chunks per input pixel

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);

    // DG 2: the first batch of this wave's filter slice (set `wave`, one set a
    // wave) goes out before the halo, so it is not queued behind the halo's
    // loads; its elements are placed while the halo streams in.  The slice
    // is contiguous in W and a multiple of 8 elements (each set's slice
    // starts on a 16-byte boundary): 16-byte chunks, kGrFB a lane a batch.
    constexpr int kGrFB = 8;
    const int dg_nel = a.bn * TAPS * a.Cg;
    const int dg_nch = DG == 2 && wave < a.gsets ? dg_nel / 8 : 0;
    i32x4 fv[kGrFB];
    auto dg_issue = [&](int c0) {
        const uint32_t gbase = uint32_t(wave) * uint32_t(dg_nel);
#pragma unroll
        for (int u = 0; u < kGrFB; ++u) {
            const int ch = c0 + u * 64 + lane;
            fv[u] = buf_load16(rw, ch < dg_nch ? (gbase + uint32_t(ch) * 8u) * 2u : kOob);
        }
    };
    if constexpr (DG == 2) dg_issue(0);

    // ---- halo: element e = pixel * cpr + stored chunk, holding source chunk
    // (stored ^ (pixel & 7)); pixels outside the image read zeros ----
    const int hchunks = a.IH * a.IW * cpr;
    for (int e0 = wave * 64; e0 < hchunks; e0 += kGrThreads) {
        const int e = e0 + lane;
        const int hp = fdiv(e, a.fd_cpr);
        const int sc = (e - hp * cpr) ^ (hp & a.hmask);
        const int ih = fdiv(hp, a.fd_iw), iw = hp - ih * a.IW;
        const int h = ho0 * s - a.pad_h + ih, w = wo0 * s - a.pad_w + iw;
        uint32_t off = kOob;
        if (e < hchunks && h >= 0 && h < a.H && w >= 0 && w < a.W)
            off = uint32_t(((n * a.H + h) * a.W + w) * a.C + sc * 8) * 2u;
        dma16(rx, hs + e0 * 16, off, 0);
    }

    const int frow = lane & 15, fgrp = lane >> 4;
    const int tile_pix = a.TH * a.TW;
    int hbase[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        int m = i * 16 + frow;
        if (m >= tile_pix) m = 0;
        const int th = fdiv(m, a.fd_tw), tw = m - th * a.TW;
        hbase[i] = th * s * a.IW + tw * s;
    }
    // weight fragments of a set: lane (frow, fgrp) of fragment (tap, j) holds
    // output channel j*16 + frow of the set against merged channels
    // fgrp*8 .. +7, zero unless those belong to that output's group
    auto load_w = [&](int gs, i32x4 (&wf)[TAPS][FN]) {
        if constexpr (DG == 2) {
            {
                // Each element of the slice (batches of chunks issued by
                // dg_issue, the first before the halo) goes into this wave's
                // part of the (not yet used) output tile in fragment order
                // [o][tap][i] (i contiguous, tap rotated).
                unsigned short* wl = reinterpret_cast<unsigned short*>(os) + wave * dg_nel;
#pragma unroll 1
                for (int c0 = 0; c0 < dg_nch; c0 += kGrFB * 64) {
                    if (c0 > 0) dg_issue(c0);
#pragma unroll
                    for (int u = 0; u < kGrFB; ++u) {
                        const int ch = c0 + u * 64 + lane;
                        if (ch < dg_nch) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) {
                                // stored order: ((gl*Cg + i)*TAPS + tap_st)*Kg + ol
                                const int e = ch * 8 + k;
                                const int q = fdiv(e, a.fd_kg), ol = e - q * a.Kg;
                                const int q2 = q / TAPS, tap_st = q - q2 * TAPS;
                                const int gl = fdiv(q2, a.fd_cg), i = q2 - gl * a.Cg;
                                wl[((gl * a.Kg + ol) * TAPS + (TAPS - 1 - tap_st)) * a.Cg + i] =
                                    static_cast<unsigned short>(uint32_t(fv[u][k >> 1]) >> (16 * (k & 1)));
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int kk = j * 16 + frow;
            const bool own = kk < a.bn && (fgrp * 8) / a.Cg == kk / a.Kg;
            if constexpr (DG == 0) {
                const uint32_t base = uint32_t(((gs * a.bn + kk) * TAPS) * a.Cg + (fgrp * 8) % a.Cg) * 2u;
#pragma unroll
                for (int tap = 0; tap < TAPS; ++tap)
                    wf[tap][j] = buf_load16(rw, own ? base + uint32_t(tap * a.Cg * 2) : kOob);
            } else if constexpr (DG == 2) {
                // fragment [tap][j] of lane (frow, fgrp): 16 bytes of the staged slice
                const int nel = a.bn * TAPS * a.Cg;
                const unsigned short* wl = reinterpret_cast<const unsigned short*>(os) + wave * nel;
                const int i0 = (fgrp * 8) % a.Cg;
#pragma unroll
                for (int tap = 0; tap < TAPS; ++tap)
                    wf[tap][j] = own ? *reinterpret_cast<const i32x4*>(wl + (kk * TAPS + tap) * a.Cg + i0)
                                     : i32x4{0, 0, 0, 0};
            } else {
                // the 8 merged channels are 8 filter rows k, TAPS * Kg elements apart
                const int o = gs * a.bn + kk;
                const int g = o / a.Kg;
                const uint32_t base = uint32_t((g * a.Cg + (fgrp * 8) % a.Cg) * TAPS * a.Kg + (o - g * a.Kg));
#pragma unroll
                for (int tap = 0; tap < TAPS; ++tap) {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        h[e] = own ? uint32_t(buf_load2(rw, (base + uint32_t((e * TAPS + TAPS - 1 - tap) * a.Kg)) * 2u))
                                   : 0u;
                    wf[tap][j] = i32x4{int(h[0] | (h[1] << 16)), int(h[2] | (h[3] << 16)),
                                       int(h[4] | (h[5] << 16)), int(h[6] | (h[7] << 16))};
                }
            }
        }
    };

    i32x4 wf[TAPS][FN];
    if (wave < a.gsets) load_w(wave, wf);
    wait_vm<0>();
    __syncthreads();

    const int out_cpr = a.K / 8;                   // 16-byte chunks per output pixel
#pragma unroll 1
    for (int gs = wave; gs < a.gsets; gs += kGrThreads / 64) {
        // (DG 2 runs one set per wave: the host picks it only when gsets <= waves)
        if constexpr (DG != 2) { if (gs != wave) load_w(gs, wf); }
        // opaque per set: keeps the per-(tap, row block) read addresses from
        // being hoisted out of the set loop (they would hold 72+ registers)
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(hbase[i]));
        f32x4 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // input fragments of a tap: all FM row blocks (rows past the tile read
        // pixel 0 and are never stored), double-buffered: the reads of tap t+1
        // are issued between the products of tap t
        i32x4 fa[2][FM];
        const uint32_t hs0 = lds_addr(hs);
        auto read_tap = [&](auto bufc, auto tapc, auto ic) {
            constexpr int B = decltype(bufc)::value, TP = decltype(tapc)::value, I = decltype(ic)::value;
            (void)fa; (void)hbase;
            const int hp = hbase[I] + (TP / S) * a.IW + TP % S;
            const uint32_t addr = hs0 + uint32_t(hp * (cpr * 16)) + uint32_t(((gs * 4 + fgrp) ^ (hp & a.hmask)) << 4);
            asm volatile("ds_read_b128 %0, %1" : "=v"(fa[B][I]) : "v"(addr));
        };
        auto wait_fa = [&](auto bufc) {
            constexpr int B = decltype(bufc)::value;
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[B][0]));
#pragma unroll
            for (int i = 1; i < FM; ++i) asm volatile("" : "+v"(fa[B][i]));
        };
        sfor<FM>([&](auto ic) { read_tap(IC<0>{}, IC<0>{}, ic); });
        wait_fa(IC<0>{});
        sfor<TAPS>([&](auto tapc) {
            constexpr int TP = decltype(tapc)::value, B = TP & 1;
            (void)fa; (void)acc; (void)wf;
            sfor<FM * FN>([&](auto mc) {
                constexpr int M = decltype(mc)::value, I = M / FN, J = M % FN;
                acc[I][J] = mfma16x16x32<T>(wf[TP][J], fa[B][I], acc[I][J]);
                if constexpr (TP + 1 < TAPS && M % FN == 0) read_tap(IC<B ^ 1>{}, IC<TP + 1>{}, IC<I>{});
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (TP + 1 < TAPS) wait_fa(IC<B ^ 1>{});
        });
        // round into the output tile: pixel m, channels gs*bn + j*16 + fgrp*4 .. +3
        // (16-byte chunk index XOR-ed by m & 15, or & 7)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = i * 16 + frow;
            if (m < tile_pix) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int col = gs * a.bn + j * 16 + fgrp * 4;
                    if (j * 16 < a.bn) {
                        const i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                                         int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
                        *reinterpret_cast<i32x2*>(os + m * (out_cpr * 16) + (((col >> 3) ^ (m & a.omask)) << 4) +
                                                  (col & 7) * 2) = v;
                    }
                }
            }
        }
    }
    __syncthreads();
    // ---- store whole output rows: element e = pixel * out_cpr + chunk ----
    const int ochunks = tile_pix * out_cpr;
    for (int e = tid; e < ochunks; e += kGrThreads) {
        const int m = fdiv(e, a.fd_kc);
        const int c = e - m * out_cpr;
        const int th = fdiv(m, a.fd_tw), tw = m - th * a.TW;
        const int ho = ho0 + th, wo = wo0 + tw;
        if (ho >= a.Ho || wo >= a.Wo) continue;
        const i32x4 v = *reinterpret_cast<const i32x4*>(os + m * (out_cpr * 16) + ((c ^ (m & a.omask)) << 4));
        buf_store16(v, ry, uint32_t(((n * a.Ho + ho) * a.Wo + wo) * a.K + c * 8) * 2u);
    }
}

// Tile geometry: up to 128 output pixels as NB whole images or TH x TW rows,
// with a halo of at most `halo_max` pixels.
bool pick_geo(const Prob& p, int halo_max, Geo* g) {
    const int64_t ho = p.ho, wo = p.wo, s = p.stride;
    auto halo = [&](int64_t nb, int64_t th, int64_t tw) {
        return nb * ((th - 1) * s + p.r) * ((tw - 1) * s + p.s);
    };
    int64_t NB = 1, TH = 1, TW = 1;
    bool whole = false;
    if (ho * wo <= kBM) {
        TH = ho; TW = wo;
        NB = std::max<int64_t>(1, std::min<int64_t>(kBM / (ho * wo), p.n));
        while (NB > 1 && halo(NB, TH, TW) > halo_max) --NB;
        whole = halo(NB, TH, TW) <= halo_max;
    }
    if (!whole) {
        // row bands of TH x TW output pixels, shrinking until the halo fits
        NB = 1;
        TW = std::min<int64_t>(wo, kBM);
        TH = std::max<int64_t>(1, std::min<int64_t>(ho, kBM / TW));
        while (TH > 1 && halo(1, TH, TW) > halo_max) --TH;
        while (TW > 8 && halo(1, TH, TW) > halo_max) TW -= 8;
    }
    if (halo(NB, TH, TW) > halo_max) return false;
    g->NB = int(NB); g->TH = int(TH); g->TW = int(TW);
    g->IH = int((TH - 1) * s + p.r);
    g->IW = int((TW - 1) * s + p.s);
    g->ptiles_n = int((p.n + NB - 1) / NB);
    g->ptiles_h = int((ho + TH - 1) / TH);
    g->ptiles_w = int((wo + TW - 1) / TW);
    return true;
}

int64_t ptiles_of(const Geo& g) { return int64_t(g.ptiles_n) * g.ptiles_h * g.ptiles_w; }

bool grouped_shape(const Prob& p, int* gm, int* bn) {
    if (p.cg > kGBK || kGBK % p.cg != 0) return false;
    const int m = int(kGBK / p.cg);
    if (p.groups % m != 0) return false;
    const int64_t n = int64_t(m) * p.kg;
    if (n % 16 != 0 || n > 64) return false;
    *gm = m;
    *bn = int(n);
    return true;
}

}  // namespace

int fwd_direct_channel_chunk() { return kBKc; }

std::string fwd_direct_reason(const Prob& p, int split_c) {
    if (fwd_window_reason(p, split_c).empty()) return "";
    if (p.cg % 8 != 0) return "input channels per group must be a multiple of 8";
    if (p.kg % 8 != 0) return "output channels per group must be a multiple of 8";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.k > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    Geo g;
    if (!pick_geo(p, kHaloMax, &g)) return "input halo of the smallest tile exceeds LDS";
    if (split_c > 1) {
        if (p.groups != 1) return "split-C needs groups == 1";
        if (p.c % split_c != 0 || (p.c / split_c) % 8 != 0)
            return "split-C needs C/split to be a multiple of 8";
    }
    return "";
}

std::string fwd_grouped_reason(const Prob& p) {
    if (p.groups < 2) return "grouped merge needs groups > 1";
    int gm, bn;
    if (!grouped_shape(p, &gm, &bn))
        return "grouped merge needs C/groups dividing 32, groups a multiple of 32/(C/groups) and "
               "(32/(C/groups))*(K/groups) a multiple of 16 up to 64";
    if (p.r * p.s > kMaxTaps) return "grouped merge stages at most 25 filter taps";
    if (p.c % 8 != 0) return "input channels must be a multiple of 8";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.k > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    Geo g;
    if (!pick_geo(p, kGHaloMax, &g)) return "input halo of the smallest tile exceeds LDS";
    return "";
}

int64_t fwd_direct_tiles(const Prob& p) {
    Geo g;
    if (!pick_geo(p, kHaloMax, &g)) return 0;
    return ptiles_of(g) * ((p.kg + kBN - 1) / kBN) * p.groups;
}

// Split the channel loop when the output alone leaves most CUs idle and there
// are enough channels to share: the largest power of two that keeps the block
// count within the CU count and at least 128 channels per split.
int fwd_direct_auto_split(const Prob& p) {
    if (p.groups != 1) return 1;
    if (fwd_window_reason(p, 1).empty()) {
        const int win = fwd_window_auto_split(p);
        // a split is wanted: small maps take the filter-streaming kernel and its split count
        if (win > 1) {
            const int sp = fwd_stream_splits(p);
            if (sp > 1 && fwd_stream_reason(p, sp).empty()) return sp;
        }
        return win;
    }
    const int64_t tiles = fwd_direct_tiles(p);
    if (tiles <= 0 || tiles >= kNumCUs / 2) return 1;
    // two blocks fit a CU (LDS), so aim for up to 2 * CUs blocks
    int best = 1;
    for (int sc = 2; sc <= 64; sc *= 2) {
        if (tiles * sc > 2 * kNumCUs) break;
        if (p.c % sc != 0 || p.c / sc < 128 || (p.c / sc) % 8 != 0) break;
        best = sc;
    }
    return best;
}

int launch_split_reduce(const Prob& p, int splits, const void* ws, void* y, hipStream_t st) {
    // 64-lane blocks: a small output still spreads over every CU
    const int64_t total4 = p.n * p.ho * p.wo * p.k / 4;
    const int64_t grid = std::min<int64_t>((total4 + 63) / 64, int64_t(kNumCUs) * 32);
    if (p.dtype == CNHWC_BF16)
        hipLaunchKernelGGL(split_reduce_kernel<BF16>, dim3(grid), dim3(64), 0, st,
                           static_cast<const float*>(ws), static_cast<unsigned short*>(y), total4,
                           total4, splits);
    else
        hipLaunchKernelGGL(split_reduce_kernel<F16>, dim3(grid), dim3(64), 0, st,
                           static_cast<const float*>(ws), static_cast<unsigned short*>(y), total4,
                           total4, splits);
    return CNHWC_OK;
}

// Direct forward (split or not): the filter-streaming kernel for split-C over
// a small map, the window kernel when it accepts the problem, else the
// register-staged kernel above.  (tune: 1 forces the register-staged kernel,
// 2 or 3 the window kernel.)
bool fwd_stream_taken(const Prob& p, const Plan& pl) {
    return pl.variant == CNHWC_VAR_FWD_SPLITC && pl.split_c > 1 && pl.tune != 1 && pl.tune != 2 &&
           pl.tune != 3 && fwd_stream_reason(p, pl.split_c).empty();
}

int launch_fwd_direct(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                      void* ws, hipStream_t st) {
    // split-C over a small map: the filter-streaming kernel (tune 3 keeps the
    // input-window kernel)
    if (fwd_stream_taken(p, pl)) return launch_fwd_stream(p, pl, x, w, y, ws, st);
    if (pl.tune != 1 && fwd_window_reason(p, pl.split_c).empty())
        return launch_fwd_window(p, pl, x, w, y, ws, st);
    if (pl.tune == 2 || pl.tune == 3) return CNHWC_UNSUPPORTED;
    FwdArgs a{};
    const bool split = pl.variant == CNHWC_VAR_FWD_SPLITC && pl.split_c > 1;
    if (!pick_geo(p, kHaloMax, &a.geo)) return CNHWC_UNSUPPORTED;
    a.x = x; a.w = w; a.y = split ? ws : y;
    a.x_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    const int64_t m = p.n * p.ho * p.wo;
    a.y_bytes = split ? uint32_t(int64_t(pl.split_c) * m * p.k * 4) : uint32_t(m * p.k * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg); a.G = p.groups;
    a.ntiles = int((p.kg + kBN - 1) / kBN);
    a.splits = split ? pl.split_c : 1;
    a.csplit = int(p.cg / a.splits);
    const int64_t blocks = ptiles_of(a.geo) * a.ntiles * a.G * a.splits;
    a.nblocks = int(blocks);
    a.remap = (blocks % 8 == 0) ? 1 : 0;
    const bool bf = p.dtype == CNHWC_BF16;
    a.halo_bytes = a.geo.NB * a.geo.IH * a.geo.IW * 128;
    const size_t stages = size_t(2) * a.halo_bytes + size_t(2) * kBN * 128;
    const size_t epi = size_t(kBM) * (kBN * (split ? 4 : 2) + 16);
    const size_t lds = std::max(stages, epi);
    const void* fn = split ? (bf ? reinterpret_cast<const void*>(&fwd_direct_kernel<BF16, true>)
                                 : reinterpret_cast<const void*>(&fwd_direct_kernel<F16, true>))
                           : (bf ? reinterpret_cast<const void*>(&fwd_direct_kernel<BF16, false>)
                                 : reinterpret_cast<const void*>(&fwd_direct_kernel<F16, false>));
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
        return CNHWC_HIP_ERROR;
    if (split) {
        if (bf) hipLaunchKernelGGL((fwd_direct_kernel<BF16, true>), dim3(blocks), dim3(kThreads), lds, st, a);
        else hipLaunchKernelGGL((fwd_direct_kernel<F16, true>), dim3(blocks), dim3(kThreads), lds, st, a);
        const int64_t total4 = m * p.k / 4;
        const int64_t grid = std::min<int64_t>((total4 + 255) / 256, int64_t(kNumCUs) * 8);
        if (bf)
            hipLaunchKernelGGL(split_reduce_kernel<BF16>, dim3(grid), dim3(256), 0, st,
                               static_cast<const float*>(ws), static_cast<unsigned short*>(y),
                               total4, total4, a.splits);
        else
            hipLaunchKernelGGL(split_reduce_kernel<F16>, dim3(grid), dim3(256), 0, st,
                               static_cast<const float*>(ws), static_cast<unsigned short*>(y),
                               total4, total4, a.splits);
    } else {
        if (bf) hipLaunchKernelGGL((fwd_direct_kernel<BF16, false>), dim3(blocks), dim3(kThreads), lds, st, a);
        else hipLaunchKernelGGL((fwd_direct_kernel<F16, false>), dim3(blocks), dim3(kThreads), lds, st, a);
    }
    return CNHWC_OK;
}

// Whole-row grouped variant: tile geometry (one image, TH x TW <= 128 output
// pixels, halo + output tile within LDS) or false when it does not apply.
static bool grow_geometry(const Prob& p, GrowArgs* a, size_t* lds) {
    int gm, bn;
    if (!grouped_shape(p, &gm, &bn)) return false;
    if (p.cg % 8 != 0 || p.c % 64 != 0 || p.k % 64 != 0) return false;
    const bool t9 = p.r == 3 && p.s == 3, t1 = p.r == 1 && p.s == 1;
    if (!(t9 && bn <= 32) && !t1) return false;
    const int64_t s = p.stride;
    int64_t TW = std::min<int64_t>(p.wo, kBM), TH = std::max<int64_t>(1, std::min<int64_t>(p.ho, kBM / TW));
    auto need = [&](int64_t th, int64_t tw) {
        const int64_t ih = (th - 1) * s + p.r, iw = (tw - 1) * s + p.s;
        const int64_t halo = (ih * iw * (p.c / 8) + 63) / 64 * 1024;
        return std::make_pair(halo, halo + th * tw * p.k * 2);
    };
    while (TH > 1 && need(TH, TW).second > 160 * 1024) --TH;
    while (TW > 8 && need(TH, TW).second > 160 * 1024) TW -= 8;
    if (need(TH, TW).second > 160 * 1024) return false;
    {
        // fewer tiles than CUs: halve the tile width and even out the rows
        const int64_t tiles = p.n * ((p.ho + TH - 1) / TH) * ((p.wo + TW - 1) / TW);
        if (tiles < kNumCUs && TW >= 16) {
            const int64_t tw2 = (TW + 1) / 2;
            const int64_t th_max = std::min<int64_t>(p.ho, kBM / tw2);
            const int64_t nth = (p.ho + th_max - 1) / th_max;
            const int64_t th2 = (p.ho + nth - 1) / nth;
            const int64_t tiles2 = p.n * nth * ((p.wo + tw2 - 1) / tw2);
            if (tiles2 <= kNumCUs && tiles2 > tiles && need(th2, tw2).second <= 160 * 1024) {
                TH = th2;
                TW = tw2;
            }
        }
    }
    a->TH = int(TH); a->TW = int(TW);
    a->IH = int((TH - 1) * s + p.r); a->IW = int((TW - 1) * s + p.s);
    a->ptiles_h = int((p.ho + TH - 1) / TH);
    a->ptiles_w = int((p.wo + TW - 1) / TW);
    a->halo_bytes = int(need(TH, TW).first);
    a->bn = bn;
    a->gsets = p.groups / gm;
    *lds = size_t(need(TH, TW).second);
    return true;
}

// p: the forward problem, or for dgrad (dg) the swapped correlation problem
static int launch_grouped_rows(const Prob& p, bool dg, const void* x, const void* w, void* y, hipStream_t st) {
    GrowArgs a{};
    size_t lds = 0;
    if (!grow_geometry(p, &a, &lds)) return CNHWC_UNSUPPORTED;
    a.x = x; a.w = w; a.y = y;
    a.x_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    a.y_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg);
    a.fd_cpr = make_fastdiv(uint32_t(p.c / 8));
    a.fd_iw = make_fastdiv(uint32_t(a.IW));
    a.fd_tw = make_fastdiv(uint32_t(a.TW));
    a.fd_kc = make_fastdiv(uint32_t(p.k / 8));
    a.hmask = (p.c / 8) % 16 == 0 ? 15 : 7;
    a.omask = (p.k / 8) % 16 == 0 ? 15 : 7;
    a.fd_kg = make_fastdiv(uint32_t(p.kg));
    a.fd_cg = make_fastdiv(uint32_t(p.cg));
    {
        // dgrad filter slices through LDS: one group set per wave, all slices
        // within the output tile's LDS, 16-byte aligned fragment reads
        const int64_t slice = int64_t(a.bn) * p.r * p.s * p.cg * 2;
        a.dg_lds = dg && a.gsets <= kGrThreads / 64 && p.cg % 8 == 0 &&
                   a.gsets * slice <= int64_t(a.TH) * a.TW * p.k * 2 ? 1 : 0;
    }
    const int64_t blocks = p.n * a.ptiles_h * a.ptiles_w;
    const bool bf = p.dtype == CNHWC_BF16;
    const void* fn;
    void (*launch)(const GrowArgs&, int64_t, size_t, hipStream_t);
#define CNHWC_GROW(T, BN, R, S, DG)                                                              \
    fn = reinterpret_cast<const void*>(&fwd_grouped_rows_kernel<T, BN, R, S, DG>);               \
    launch = [](const GrowArgs& g, int64_t nb, size_t l, hipStream_t q) {                        \
        hipLaunchKernelGGL((fwd_grouped_rows_kernel<T, BN, R, S, DG>), dim3(nb), dim3(kGrThreads), l, q, g); \
    };
#define CNHWC_GROW_DG(T, BN, R, S) if (dg && a.dg_lds) { CNHWC_GROW(T, BN, R, S, 2) } \
    else if (dg) { CNHWC_GROW(T, BN, R, S, 1) } else { CNHWC_GROW(T, BN, R, S, 0) }
    if (p.r == 3) {
        if (bf) { CNHWC_GROW_DG(BF16, 32, 3, 3) } else { CNHWC_GROW_DG(F16, 32, 3, 3) }
    } else if (a.bn <= 32) {
        if (bf) { CNHWC_GROW_DG(BF16, 32, 1, 1) } else { CNHWC_GROW_DG(F16, 32, 1, 1) }
    } else {
        if (bf) { CNHWC_GROW_DG(BF16, 64, 1, 1) } else { CNHWC_GROW_DG(F16, 64, 1, 1) }
    }
#undef CNHWC_GROW_DG
#undef CNHWC_GROW
    if (lds > 64 * 1024 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
        return CNHWC_HIP_ERROR;
    launch(a, blocks, lds, st);
    return CNHWC_OK;
}

int launch_fwd_grouped(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                       hipStream_t st) {
    // whole-row variant where it applies (tune 1 asks for the group-set kernel)
    if (pl.tune != 1) {
        GrowArgs g{};
        size_t lds = 0;
        if (grow_geometry(p, &g, &lds)) return launch_grouped_rows(p, false, x, w, y, st);
    }
    GrpArgs a{};
    if (!pick_geo(p, kGHaloMax, &a.geo)) return CNHWC_UNSUPPORTED;
    if (!grouped_shape(p, &a.gm, &a.bn)) return CNHWC_UNSUPPORTED;
    a.x = x; a.w = w; a.y = y;
    a.x_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    a.y_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg); a.G = p.groups;
    a.gsets = p.groups / a.gm;
    const int64_t blocks = ptiles_of(a.geo) * a.gsets;
    a.nblocks = int(blocks);
    a.remap = (blocks % 8 == 0) ? 1 : 0;
    const bool bf = p.dtype == CNHWC_BF16;
    // the halo is filled 16 pixels per load: round its LDS up to whole loads
    a.halo_bytes = (a.geo.NB * a.geo.IH * a.geo.IW + 15) / 16 * 16 * 64;
    a.fd_img = make_fastdiv(uint32_t(a.geo.IH * a.geo.IW));
    a.fd_iw = make_fastdiv(uint32_t(a.geo.IW));
    a.fd_per = make_fastdiv(uint32_t(a.geo.TH * a.geo.TW));
    a.fd_tw = make_fastdiv(uint32_t(a.geo.TW));
#define CNHWC_GRP(BNV)                                                                          \
    if (a.bn <= BNV) {                                                                          \
        const size_t lds = std::max(size_t(a.halo_bytes) + size_t(p.r * p.s) * BNV * 64,       \
                                    size_t(kBM) * (BNV * 2 + 16));  /* epilogue tile */       \
        const void* fn = bf ? reinterpret_cast<const void*>(&fwd_grouped_kernel<BF16, BNV>)     \
                            : reinterpret_cast<const void*>(&fwd_grouped_kernel<F16, BNV>);     \
        if (lds > 64 * 1024 &&                                                                  \
            hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess) \
            return CNHWC_HIP_ERROR;                                                             \
        if (bf) hipLaunchKernelGGL((fwd_grouped_kernel<BF16, BNV>), dim3(blocks), dim3(kThreads), lds, st, a); \
        else hipLaunchKernelGGL((fwd_grouped_kernel<F16, BNV>), dim3(blocks), dim3(kThreads), lds, st, a);     \
        return CNHWC_OK;                                                                        \
    }
    CNHWC_GRP(32)
    CNHWC_GRP(64)
#undef CNHWC_GRP
    return CNHWC_UNSUPPORTED;
}

// ---- grouped dgrad, stride 1, on the whole-row grouped kernel -------------
// dX is dY correlated with the filter rotated by 180 degrees and transposed
// per group (dX channel c of group g gathers dY channels g*Kg .. +Kg), at
// padding R-1-pad: a grouped forward correlation with input dY (K channels,
// Kg per group, extents Ho x Wo) and output dX (C channels, Cg per group,
// extents H x W) -- the same block-diagonal merge of small groups.
static Prob dgrad_as_fwd(const Prob& p) {
    Prob q = p;
    q.h = p.ho; q.w = p.wo; q.ho = p.h; q.wo = p.w;
    q.c = p.k; q.k = p.c; q.cg = p.kg; q.kg = p.cg;
    q.pad_h = int(p.r) - 1 - p.pad_h;
    q.pad_w = int(p.s) - 1 - p.pad_w;
    return q;
}

std::string dgrad_grouped_reason(const Prob& p) {
    if (p.groups < 2) return "grouped merge needs groups > 1";
    if (p.stride != 1) return "grouped dgrad merge needs stride 1";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.k > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    GrowArgs g{};
    size_t lds = 0;
    if (!grow_geometry(dgrad_as_fwd(p), &g, &lds))
        return "grouped dgrad merge needs K/groups dividing 32 (a multiple of 8), C and K multiples of "
               "64, a 3x3 filter with (32/(K/groups))*(C/groups) <= 32 or a 1x1 filter with it <= 64, "
               "and a tile within LDS";
    return "";
}

int launch_dgrad_grouped(const Prob& p, const Plan&, const void* dy, const void* w, void* dx,
                         hipStream_t st) {
    return launch_grouped_rows(dgrad_as_fwd(p), true, dy, w, dx, st);
}

}  // namespace cnhwc
