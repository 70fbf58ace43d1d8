// Direct forward convolution with the input window staged in LDS, pipelined
// for the gfx950 matrix cores ("feat(rocke): split-C and grouped LDS-halo
// direct conv fwd kernels": the direct kernel and its split-C form).
//
// A block owns NB images x TH rows x TW columns of output pixels (<= 224, the
// MFMA M side) and BN output channels of one group.  Per 64-channel chunk of
// its input channels, the input window those pixels reach -- per image
// ((TH-1)*s + R) x ((TW-1)*s + S) pixels, the halo -- is loaded into LDS once
// and every filter tap reads a shifted view of it.  The window is stored as 8
// planes, one per 16-byte group of 8 channels, each a dense array of window
// pixels: a tap shift is a uniform offset of every lane's read address and the
// 16 lanes of an MFMA row group read 16 consecutive 16-byte entries.  The
// weight rows of a tap (BN output channels x 64 input channels, input channels
// contiguous -- already the MFMA reduction layout) stream through a 4-stage
// LDS ring.  Both operands go global -> LDS with asynchronous loads that write
// LDS directly.
//
// The block runs 8 waves: two groups of 2 x 2 waves compute the same output
// tile over alternate reduction steps (chunk-outer, tap-inner), so each SIMD
// has two matrix-core waves whose LDS reads overlap each other's MFMAs; the
// groups' fp32 sums are added at the end.
//
// Split-C: the channel loop is divided among blocks (grid axis = split index);
// each block writes its fp32 partial tile to a workspace [split][pixel][K] and
// the reduce pass of the direct-forward file sums the splits in ascending
// order and rounds once.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>

namespace cnhwc {
namespace {

constexpr int kThreads = 512;
constexpr int kBK = 64;           // input channels per reduction step
constexpr int kRing = 4;          // weight ring stages
constexpr int kMaxQ = 7;          // 64-pixel groups per window plane
constexpr int kLdsMax = 160 * 1024;
constexpr int kBMC = 224;         // tile capacity in pixels (2 x 7 MFMA row tiles)

struct WinGeo {
    int NB, TH, TW;               // tile: images x rows x columns
    int IH, IW;                   // window rows / columns per image
    int hp;                       // window plane entries (multiple of 64)
    int tiles_n, tiles_h, tiles_w;
    FastDiv fd_img, fd_iw, fd_per, fd_tw;   // division by IH*IW, IW, TH*TW, TW
};

struct FwinArgs {
    const void* x;
    const void* w;
    void* y;                      // output, or the fp32 workspace when split
    uint32_t x_bytes, w_bytes, y_bytes;
    int N, H, W, C, K, R, S, stride, pad_h, pad_w, Ho, Wo, Cg, Kg, G;
    WinGeo geo;
    int ntiles;                   // output-channel tiles per group
    int splits, csplit;           // channel splits and channels per split
    int nblocks, remap;
    uint32_t halo_bytes;          // one window buffer (8 planes x hp x 16 bytes)
};

template <typename T, int WNB, bool SPLIT, bool KR>
__global__ __launch_bounds__(kThreads, 1) void fwd_window_kernel(const FwinArgs a) {
    constexpr int WMB = kBMC / 32;                      // 7 row tiles per wave
    constexpr int BN = 2 * WNB * 16;                    // output channels per tile
    constexpr int B_BYTES = BN * 128;                   // one ring stage: BN rows x 64 channels
    constexpr int B_REG = B_BYTES / 1024 / 4;           // loads per lane per stage (4 waves)
    constexpr int ESZ = SPLIT ? 4 : 2;
    constexpr int C_STRIDE = BN * ESZ + 16;
    static_assert(B_BYTES % 4096 == 0, "stage splits over 4 waves");
    static_assert(3 * B_BYTES + 128 < 65536, "stage offsets fit the LDS immediate");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int lw = wave & 3;
    const WinGeo& geo = a.geo;

    // ---- block -> (output tile, channel tile, group, split) ----
    int bid = blockIdx.x;
    if (a.remap) bid = (bid & 7) * (a.nblocks >> 3) + (bid >> 3);
    const int nt = bid % a.ntiles;
    int rest = bid / a.ntiles;
    const int ptiles = geo.tiles_n * geo.tiles_h * geo.tiles_w;
    const int pt = rest % ptiles;
    rest /= ptiles;
    const int g = rest % a.G;
    const int sp = rest / a.G;
    const int tw_i = pt % geo.tiles_w;
    const int th_i = (pt / geo.tiles_w) % geo.tiles_h;
    const int n0 = (pt / (geo.tiles_w * geo.tiles_h)) * geo.NB;
    const int ho0 = th_i * geo.TH, wo0 = tw_i * geo.TW;
    const int k0 = nt * BN;                              // within the group
    const int c_lo = sp * a.csplit;                      // within the group
    const int c_hi = min(a.Cg, c_lo + a.csplit);
    const int s = a.stride;
    const int hp = geo.hp;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.y, a.y_bytes);

    // ---- per-lane window sources: lane covers window pixel i*64 + lane ----
    const int per_img = geo.IH * geo.IW;
    const int hreal = geo.NB * per_img;
    const int nq = hp >> 6;
    uint32_t hoff[kMaxQ];
#pragma unroll
    for (int i = 0; i < kMaxQ; ++i) {
        const int q = i * 64 + lane;
        hoff[i] = kOob;
        if (i < nq && q < hreal) {
            const int nb = fdiv(q, geo.fd_img);
            const int rem = q - nb * per_img;
            const int iy = fdiv(rem, geo.fd_iw);
            const int ix = rem - iy * geo.IW;
            const int n = n0 + nb;
            const int h = ho0 * s - a.pad_h + iy, w = wo0 * s - a.pad_w + ix;
            if (n < a.N && h >= 0 && h < a.H && w >= 0 && w < a.W)
                hoff[i] = uint32_t((((n * a.H + h) * a.W + w) * a.C + g * a.Cg + c_lo) * 2);
        }
    }
    // window of chunk cc into buffer buf: wave w fills plane w
    auto issue_window = [&](int buf, int cc) {
        const int c = cc * kBK + wave * 8;               // channel offset within the split
        unsigned char* base = lds + buf * a.halo_bytes + wave * hp * 16;
        const uint32_t soff = uint32_t(c * 2);
        const bool cin = !KR || c_lo + c < c_hi;
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i)
            if (i < nq) dma16(rx, base + i * 1024, cin ? hoff[i] : kOob, soff);
    };

    // ---- per-lane weight sources: a group's 4 waves fill one stage ----
    // region E of wave lw holds rows 8*(lw + 4E) .. +7; lane -> (row, 16-byte
    // chunk); physical chunk = logical ^ (row & 7)
    const int taps = a.R * a.S;
    const int wrow_stride = taps * a.Cg;                 // elements between weight rows
    uint32_t b_voff[B_REG];
#pragma unroll
    for (int e = 0; e < B_REG; ++e) {
        const int row = 8 * (lw + 4 * e) + (lane >> 3);
        const int chunk = (lane & 7) ^ (row & 7);
        b_voff[e] = k0 + row < a.Kg ? uint32_t((row * wrow_stride + chunk * 8) * 2) : kOob;
    }

    const int cchunks = (c_hi - c_lo + kBK - 1) / kBK;
    const int steps = taps * cchunks;
    const bool defer1 = taps >= 4;
    unsigned char* const ring_g = lds + 2 * a.halo_bytes + grp * B_BYTES;

    // weight issue cursor of this group: tap wt, chunk wc
    int wt = 0, wc = 0;
    auto advance_w = [&]() {
        ++wt;
        const bool w1 = wt >= taps;
        wt = w1 ? 0 : wt;
        wc += w1 ? 1 : 0;
    };
    auto dma_w = [&](auto stg, auto ec) {
        constexpr int STG = decltype(stg)::value, E = decltype(ec)::value;
        (void)b_voff;
        const uint32_t soff =
            uint32_t((((g * a.Kg + k0) * taps + wt) * a.Cg + c_lo + wc * kBK) * 2);
        uint32_t v = b_voff[E];
        if (KR) {
            const int row = 8 * (lw + 4 * E) + (lane >> 3);
            const int chunk = (lane & 7) ^ (row & 7);
            v = (c_lo + wc * kBK + chunk * 8 < c_hi) ? v : kOob;
        }
        dma16(rw, ring_g + STG * B_BYTES + (lw + 4 * E) * 1024, v, soff);
    };

    // ---- fragment read addresses ----
    const int wm = lw >> 1, wn = lw & 1;
    const int frow = lane & 15, fgrp = lane >> 4;
    const uint32_t lds0 = lds_addr(lds);
    const int tpix = geo.NB * geo.TH * geo.TW;
    uint32_t fa_base[WMB];               // window buffer 0, half 0, tap (0, 0)
#pragma unroll
    for (int i = 0; i < WMB; ++i) {
        int m = wm * (WMB * 16) + i * 16 + frow;
        if (m >= tpix) m = 0;
        const int per = geo.TH * geo.TW;
        const int nb = fdiv(m, geo.fd_per);
        const int rem = m - nb * per;
        const int y = fdiv(rem, geo.fd_tw), x = rem - y * geo.TW;
        const int q = nb * per_img + y * s * geo.IW + x * s;
        fa_base[i] = lds0 + uint32_t((fgrp * hp + q) * 16);
    }
    uint32_t fb_addr[2][WNB];            // this group's first ring stage
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < WNB; ++j) {
            const int row = wn * (WNB * 16) + j * 16 + frow;
            fb_addr[ks][j] = lds_addr(ring_g) + row * 128 + (((ks * 4 + fgrp) ^ (row & 7)) << 4);
        }
    const int plane4 = 4 * hp * 16;

    // read cursor of this group: tap rt, chunk rc of the own step whose first
    // half is read next; offset = window buffer + tap shift
    int rr = 0, rs = 0, rc = 0;
    auto cursor_off = [&]() {
        return (rc & 1) * int(a.halo_bytes) + (rr * geo.IW + rs) * 16;
    };
    auto advance_r = [&]() {
        ++rs;
        const bool w1 = rs >= a.S;
        rs = w1 ? 0 : rs;
        rr += w1 ? 1 : 0;
        const bool w2 = rr >= a.R;
        rr = w2 ? 0 : rr;
        rc += w2 ? 1 : 0;
    };

    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 fa[2][WMB], fb[2][WNB];
    constexpr int NREAD = WNB + WMB;
    auto read_one = [&](auto stg, auto ksc, auto rcc, int aoff) {
        constexpr int STG = decltype(stg)::value, KS = decltype(ksc)::value;
        constexpr int R = decltype(rcc)::value;
        (void)fa; (void)fb; (void)fa_base; (void)fb_addr; (void)plane4;
        if constexpr (R < WNB) {
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(fb[KS][R]) : "v"(fb_addr[KS][R]), "i"(STG * B_BYTES));
        } else {
            asm volatile("ds_read_b128 %0, %1"
                         : "=v"(fa[KS][R - WNB])
                         : "v"(fa_base[R - WNB] + uint32_t(aoff + KS * plane4)));
        }
    };
    auto wait_frags = [&](auto ksc) {
        constexpr int KS = decltype(ksc)::value;
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[KS][0]), "+v"(fb[KS][0]));
#pragma unroll
        for (int i = 1; i < WMB; ++i) asm volatile("" : "+v"(fa[KS][i]));
#pragma unroll
        for (int j = 1; j < WNB; ++j) asm volatile("" : "+v"(fb[KS][j]));
    };
    auto mfma_one = [&](auto ksc, auto mc) {
        constexpr int KS = decltype(ksc)::value, M = decltype(mc)::value;
        constexpr int i = M / WNB, j = M % WNB;
        // rows = output channels (weights), columns = pixels (input window)
        acc[i][j] = mfma16x16x32<T>(fb[KS][j], fa[KS][i], acc[i][j]);
    };

    constexpr int NM = WMB * WNB;
    constexpr int PER0 = (NREAD + NM - 1) / NM;
    constexpr int NI1 = NREAD + B_REG;
    constexpr int PER1 = (NI1 + NM - 1) / NM;
    int off_cur = 0, off_next = 0;
    int end_step = taps - 1;             // last step of chunk end_chunk (block-uniform)
    int end_chunk = 0;
    // Super-step j: group g multiplies its step 2j + g.  First half: multiply
    // half 0 while reading half 1.  Every wave then waits for its own loads
    // and all meet at the barrier.  Second half: multiply half 1 while loading
    // the group's step after next into the stage just freed and reading half
    // 0 of its next step.  A chunk whose last step was in this super-step
    // frees its window buffer for the chunk after next.
    auto super_fn = [&](auto jc, int j) {
        constexpr int J = decltype(jc)::value;
        constexpr int STG = 2 * J, NXT = 2 * (1 - J);
        const bool active = 2 * j + grp < steps;
        if (active) {
            sfor<NM>([&](auto mc) {
                constexpr int M = decltype(mc)::value;
                mfma_one(IC<0>{}, mc);
                sfor<PER0>([&](auto pc) {
                    constexpr int X = M * PER0 + decltype(pc)::value;
                    if constexpr (X < NREAD) read_one(IC<STG>{}, IC<1>{}, IC<X>{}, off_cur);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        wait_frags(IC<1>{});
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (active) {
            sfor<NM>([&](auto mc) {
                constexpr int M = decltype(mc)::value;
                mfma_one(IC<1>{}, mc);
                sfor<PER1>([&](auto pc) {
                    constexpr int X = M * PER1 + decltype(pc)::value;
                    if constexpr (X < B_REG) dma_w(IC<STG>{}, IC<X>{});
                    else if constexpr (X < NI1) read_one(IC<NXT>{}, IC<0>{}, IC<X - B_REG>{}, off_next);
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        if (defer1 && j == 0) issue_window(1, 1);
        if (end_step <= 2 * j + 1) {
            issue_window(end_chunk & 1, end_chunk + 2);
            ++end_chunk;
            end_step += taps;
        }
        wait_frags(IC<0>{});
        off_cur = off_next;
        advance_r();
        advance_r();
        off_next = cursor_off();
        advance_w();
        advance_w();
    };

    if (steps > 0) {
        issue_window(0, 0);
        if (grp) advance_w();
        sfor<B_REG>([&](auto ec) { dma_w(IC<0>{}, ec); });
        advance_w();
        advance_w();
        if (!defer1) issue_window(1, 1);
        sfor<B_REG>([&](auto ec) { dma_w(IC<2>{}, ec); });
        advance_w();
        advance_w();
        wait_vm<B_REG>();
        __builtin_amdgcn_s_barrier();
        if (grp) advance_r();
        off_cur = cursor_off();
        advance_r();
        advance_r();
        off_next = cursor_off();
        sfor<NREAD>([&](auto rcc) { read_one(IC<0>{}, IC<0>{}, rcc, off_cur); });
        wait_frags(IC<0>{});
        const int supers = (steps + 1) / 2;
#pragma unroll 1
        for (int j = 0; j < supers; j += 2) {
            super_fn(IC<0>{}, j);
            if (j + 1 < supers) super_fn(IC<1>{}, j + 1);
        }
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
    }

    // ---- add the odd-step partials into the even-step group's ----
    f32x4* part = reinterpret_cast<f32x4*>(lds) + lw * NM * 64 + lane;
    if (grp == 1) {
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j) part[(i * WNB + j) * 64] = acc[i][j];
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j) acc[i][j] += part[(i * WNB + j) * 64];
    }
    __syncthreads();

    // ---- epilogue: stage the tile in LDS (fp32 or rounded), 16-byte stores ----
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j) {
                const int row = wm * (WMB * 16) + i * 16 + frow;
                const int col = wn * (WNB * 16) + j * 16 + fgrp * 4;
                if constexpr (SPLIT) {
                    *reinterpret_cast<f32x4*>(lds + row * C_STRIDE + col * 4) = acc[i][j];
                } else {
                    i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                               int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
                    *reinterpret_cast<i32x2*>(lds + row * C_STRIDE + col * 2) = v;
                }
            }
    }
    __syncthreads();
    constexpr int CPR = BN * ESZ / 16;
    const int mtotal = a.N * a.Ho * a.Wo;
    const int per = geo.TH * geo.TW;
    for (int q = tid; q < kBMC * CPR; q += kThreads) {
        const int row = q / CPR, cc = q % CPR;
        if (row >= tpix) continue;
        const int nb = fdiv(row, geo.fd_per);
        const int rem = row - nb * per;
        const int y = fdiv(rem, geo.fd_tw), x = rem - y * geo.TW;
        const int n = n0 + nb, ho = ho0 + y, wo = wo0 + x;
        if (n >= a.N || ho >= a.Ho || wo >= a.Wo) continue;
        const int kl = k0 + cc * (16 / ESZ);
        if (kl >= a.Kg) continue;
        const int pix = (n * a.Ho + ho) * a.Wo + wo;
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + row * C_STRIDE + cc * 16);
        if constexpr (SPLIT)
            buf_store16(v, ry, uint32_t(((sp * mtotal + pix) * a.K + g * a.Kg + kl) * 4));
        else
            buf_store16(v, ry, uint32_t((pix * a.K + g * a.Kg + kl) * 2));
    }
}

// Window plane entries one buffer may hold next to a BN-channel weight ring.
int win_hp_max(int bn) {
    return std::min(kMaxQ * 64, (kLdsMax - kRing * bn * 128) / (2 * 8 * 16) / 64 * 64);
}

// Tile shape: whole images when several fit the 224-pixel capacity, else row
// bands of the full output width (or column bands), shrunk until the window
// fits; th_cap limits the rows of a band.
bool win_geo(const Prob& p, int bn, int th_cap, WinGeo* g) {
    const int64_t ho = p.ho, wo = p.wo, s = p.stride;
    const int hp_max = win_hp_max(bn);
    auto window = [&](int64_t nb, int64_t th, int64_t tw) {
        return nb * ((th - 1) * s + p.r) * ((tw - 1) * s + p.s);
    };
    int64_t NB = 1, TH = 1, TW = 1;
    bool whole = false;
    if (ho * wo <= kBMC && ho <= th_cap) {
        TH = ho; TW = wo;
        NB = std::max<int64_t>(1, std::min<int64_t>(kBMC / (ho * wo), p.n));
        while (NB > 1 && window(NB, TH, TW) > hp_max) --NB;
        whole = window(NB, TH, TW) <= hp_max;
    }
    if (!whole) {
        NB = 1;
        TW = std::min<int64_t>(wo, kBMC);
        TH = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(ho, kBMC / TW), th_cap));
        while (TH > 1 && window(1, TH, TW) > hp_max) --TH;
        while (TW > 8 && window(1, TH, TW) > hp_max) TW -= 8;
        while (TW > 1 && window(1, TH, TW) > hp_max) --TW;
    }
    if (window(NB, TH, TW) > hp_max) return false;
    g->NB = int(NB); g->TH = int(TH); g->TW = int(TW);
    g->IH = int((TH - 1) * s + p.r);
    g->IW = int((TW - 1) * s + p.s);
    g->hp = int((window(NB, TH, TW) + 63) / 64 * 64);
    g->tiles_n = int((p.n + NB - 1) / NB);
    g->tiles_h = int((ho + TH - 1) / TH);
    g->tiles_w = int((wo + TW - 1) / TW);
    g->fd_img = make_fastdiv(uint32_t(g->IH * g->IW));
    g->fd_iw = make_fastdiv(uint32_t(g->IW));
    g->fd_per = make_fastdiv(uint32_t(g->TH * g->TW));
    g->fd_tw = make_fastdiv(uint32_t(g->TW));
    return true;
}

int64_t win_tiles(const WinGeo& g) { return int64_t(g.tiles_n) * g.tiles_h * g.tiles_w; }

// Output channels per tile: 128 when that alone gives every CU a block, else
// 64 (more, smaller tiles for small outputs, so fewer channel splits).
int win_bn(const Prob& p) {
    if (p.kg <= 64) return 64;
    WinGeo g;
    if (!win_geo(p, 128, kBMC, &g)) return 64;
    return win_tiles(g) * ((p.kg + 127) / 128) * p.groups >= kNumCUs ? 128 : 64;
}

// Row cap minimising rounds of blocks over the CUs (one block per CU).
bool win_best_geo(const Prob& p, int splits, WinGeo* best) {
    const int bn = win_bn(p);
    const int64_t ntiles = (p.kg + bn - 1) / bn;
    int64_t best_rounds = INT64_MAX;
    bool found = false;
    for (int cap = kBMC; cap >= 1; --cap) {
        WinGeo g;
        if (!win_geo(p, bn, cap, &g)) continue;
        const int64_t blocks = win_tiles(g) * ntiles * p.groups * splits;
        const int64_t rounds = (blocks + kNumCUs - 1) / kNumCUs;
        if (rounds < best_rounds) { best_rounds = rounds; *best = g; found = true; }
        if (g.TH < cap && g.NB == 1 && cap > g.TH) cap = g.TH + 1;   // skip caps that change nothing
    }
    return found;
}

template <typename T, int WNB, bool SPLIT, bool KR>
int launch_inst(const FwinArgs& a, size_t lds, hipStream_t st) {
    auto kern = fwd_window_kernel<T, WNB, SPLIT, KR>;
    static bool attr_set = false;   // the attribute is per kernel; idempotent if raced
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess)
            return CNHWC_HIP_ERROR;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(a.nblocks), dim3(kThreads), lds, st, a);
    return CNHWC_OK;
}

template <typename T, int WNB>
int launch_t(bool split, bool kr, const FwinArgs& a, size_t lds, hipStream_t st) {
    if (split) return kr ? launch_inst<T, WNB, true, true>(a, lds, st)
                         : launch_inst<T, WNB, true, false>(a, lds, st);
    return kr ? launch_inst<T, WNB, false, true>(a, lds, st)
              : launch_inst<T, WNB, false, false>(a, lds, st);
}

}  // namespace

std::string fwd_window_reason(const Prob& p, int split_c) {
    if (p.cg % 8 != 0) return "input channels per group must be a multiple of 8";
    if (p.kg % 8 != 0) return "output channels per group must be a multiple of 8";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.k > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    WinGeo g;
    if (!win_geo(p, win_bn(p), kBMC, &g)) return "input window of the smallest tile exceeds LDS";
    if (split_c > 1) {
        if (p.groups != 1) return "split-C needs groups == 1";
        if (p.c % split_c != 0 || (p.c / split_c) % 8 != 0)
            return "split-C needs C/split to be a multiple of 8";
    }
    return "";
}

// Splits for the window kernel: the largest power of two that keeps the block
// count within the CU count (one block per CU) with >= 128 channels a split.
int fwd_window_auto_split(const Prob& p) {
    if (p.groups != 1) return 1;
    WinGeo g;
    if (!win_best_geo(p, 1, &g)) return 1;
    const int64_t tiles = win_tiles(g) * ((p.kg + win_bn(p) - 1) / win_bn(p));
    if (tiles >= kNumCUs / 2) return 1;
    int best = 1;
    for (int sc = 2; sc <= 64; sc *= 2) {
        if (tiles * sc > kNumCUs) break;
        if (p.c % sc != 0 || p.c / sc < 128 || (p.c / sc) % 8 != 0) break;
        best = sc;
    }
    return best;
}

int launch_fwd_window(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                      void* ws, hipStream_t st) {
    const bool split = pl.variant == CNHWC_VAR_FWD_SPLITC && pl.split_c > 1;
    const int splits = split ? pl.split_c : 1;
    FwinArgs a{};
    if (!win_best_geo(p, splits, &a.geo)) return CNHWC_UNSUPPORTED;
    const int bn = win_bn(p);
    a.x = x; a.w = w; a.y = split ? ws : y;
    a.x_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    const int64_t m = p.n * p.ho * p.wo;
    a.y_bytes = split ? uint32_t(int64_t(splits) * m * p.k * 4) : uint32_t(m * p.k * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg); a.G = p.groups;
    a.ntiles = int((p.kg + bn - 1) / bn);
    a.splits = splits;
    a.csplit = int(p.cg / splits);
    const int64_t blocks = win_tiles(a.geo) * a.ntiles * a.G * splits;
    a.nblocks = int(blocks);
    a.remap = (blocks % 8 == 0) ? 1 : 0;
    a.halo_bytes = uint32_t(8 * a.geo.hp * 16);
    const size_t ring = size_t(kRing) * bn * 128;
    const size_t epi = size_t(kBMC) * (bn * (split ? 4 : 2) + 16);
    const size_t partials = size_t(kBMC) * bn * 4;
    const size_t lds = std::max(std::max(2 * size_t(a.halo_bytes) + ring, epi), partials);
    const bool kr = a.csplit % kBK != 0;
    const bool bf = p.dtype == CNHWC_BF16;
    int rc;
    if (bn == 128) rc = bf ? launch_t<BF16, 4>(split, kr, a, lds, st) : launch_t<F16, 4>(split, kr, a, lds, st);
    else rc = bf ? launch_t<BF16, 2>(split, kr, a, lds, st) : launch_t<F16, 2>(split, kr, a, lds, st);
    if (rc != CNHWC_OK || !split) return rc;
    return launch_split_reduce(p, splits, ws, y, st);
}

}  // namespace cnhwc
