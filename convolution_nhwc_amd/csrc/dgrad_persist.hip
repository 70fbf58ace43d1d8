// Strided dgrad on a persistent 8-wave implicit-GEMM kernel.
//
// The arithmetic is that of the ring kernel in dgrad_igemm.hip: dX splits
// into stride*stride phase classes (the "tilde" decomposition of
// "perf(rocke/conv): add the pointwise fast path dgrad was missing", Finding 4
// and the fast-path commit); class (a, b) is the dense GEMM
//     dX_class[m, c] = sum_{i, j, k} dY[n, u0(m) - i, v0(m) - j, g*Kg + k] * W[g*Kg + k, r0 + s*i, t0 + s*j, c]
// and every output runs the same chain of 32-deep MFMA steps in the same
// order (taps outer, k inner), so both kernels give the same bits.
//
// What differs is the schedule.  Strided classes have few taps, so a block of
// the ring kernel runs only 4-16 reduction steps and its set-up, first loads
// and output stores -- about half its life -- are exposed, in several rounds
// of blocks that move in lockstep.  Here:
//   * One block per CU, 8 waves (two per SIMD) on a 224-pixel x 256-channel
//     tile: 2 x 4 waves of 112 pixels x 64 channels (7 x 4 MFMA 16x16x32).
//     A 32-deep step needs 30 KiB of operands for 3.7 MFLOP.
//   * Each class gets its own set of blocks, sized so that every block runs
//     about the same number of reduction steps (a class with half the taps
//     gets half the blocks per tile); a block walks a contiguous range of its
//     class's tiles, so it never changes class.
//   * One ring of 4 stages (32-deep dY and W slices) runs through all of a
//     block's tiles: the loads of a tile's first steps are in flight while the
//     previous tile is multiplied.  A finished tile is rounded (RNE) and
//     stored from the accumulators at the start of the next tile's first step
//     (a cross-row lane swap gives each lane 8 consecutive channels, so the 4
//     lanes of a pixel store 64 contiguous bytes); the block's last tile goes
//     through a small per-wave LDS staging area as whole 128-byte rows.
//   * A step: wait for the next stage, one barrier, then 28 MFMAs per wave
//     with the next step's 15 fragment reads and the loads of the step three
//     ahead placed between them.
//
// LDS: A stages hold 224 rows of 64 bytes (one pixel's 32 channels of dY; the
// four 16-byte chunks of row q stored at chunk ^ ((q >> 2) & 3)); W stages
// hold 32 k-rows of 512 bytes (256 channels; 16-byte chunk pairs XOR-ed per
// row, read with the LDS transpose read).  The swizzles are applied through
// the load source addresses.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <cstddef>
#include <string>
#include <type_traits>

namespace cnhwc {
namespace {

constexpr int kPThreads = 512;
constexpr int kPBK = 32;                   // reduction depth per stage
constexpr int kPWMB = 7, kPWNB = 4;        // 16x16 tiles per wave: pixels, channels
constexpr int kPBM = 2 * kPWMB * 16;       // 224 pixels per tile
constexpr int kPBN = 4 * kPWNB * 16;       // 256 channels per tile
constexpr int kPStages = 4;
constexpr int kPARow = kPBK * 2;           // 64 bytes
constexpr int kPABytes = kPBM * kPARow;    // one dY stage: 14 KiB
constexpr int kPBRow = kPBN * 2;           // 512 bytes
constexpr int kPBBytes = kPBK * kPBRow;    // one W stage: 16 KiB
constexpr int kPBBase = kPStages * kPABytes;
constexpr int kPLds = kPStages * (kPABytes + kPBBytes);   // 120 KiB of stages
constexpr int kPEpiWave = 16 * 128;        // epilogue staging per wave: 16 pixels x 128 bytes
constexpr int kPARegs = kPABytes / 1024;   // 14 one-KiB regions of 16 pixel rows
constexpr int kPBRegs = kPBBytes / 1024;   // 16 regions of 2 k-rows
constexpr int kPMaxClasses = 16;
constexpr int kPPre = 2;                   // pixel tiles multiplied before a step's barrier
constexpr int kPTail = 2;                  // dY reads left in flight across a step boundary
static_assert((kPWMB - kPPre) * (kPWNB - 1) >= 2 * kPWNB + 4, "gaps for the W reads and the loads");

// LDS reads a step issues before its first load (the schedule of the step
// below: kPPre dY reads after the barrier, then per product a dY read after
// the fourth product of a pixel tile and W reads in the other gaps)
constexpr int p_lds_before_loads() {
    int n = kPPre;
    for (int m = kPPre * kPWNB; m < kPWMB * kPWNB; ++m) {
        const int i = m / kPWNB, j = m % kPWNB;
        if (j == kPWNB - 1) { ++n; continue; }
        const int q = (i - kPPre) * (kPWNB - 1) + j;
        if (q < 2 * kPWNB) ++n;
        else return n;
    }
    return n;
}
// product index after which the last load of a step issues
constexpr int p_last_load() {
    int last = -1;
    for (int m = kPPre * kPWNB; m < kPWMB * kPWNB; ++m) {
        const int i = m / kPWNB, j = m % kPWNB;
        if (j == kPWNB - 1) continue;
        const int q = (i - kPPre) * (kPWNB - 1) + j;
        if (q >= 2 * kPWNB && q < 2 * kPWNB + 4) last = m;
    }
    return last;
}
// the tail reads (the dY reads after the fourth product of pixel tiles
// kPWMB-2 and kPWMB-1) are a step's last two LDS operations and come after
// its loads
static_assert(kPTail == 2 && (kPWMB - kPTail) * kPWNB + kPWNB - 1 > p_last_load(), "tail reads after the loads");
static_assert(kPBRegs == 16 && kPARegs > 8 && kPARegs <= 16, "two regions of each operand per wave");
static_assert((kPStages - 1) * kPBBytes < 65536, "stage offsets fit the LDS immediate");

struct PClass {
    int a, b;            // phase: h = a + s*hc, w = b + s*wc
    int hc, wc;          // rows / columns of dX in the class
    int r0, t0, nr, nt;  // first filter row / column and how many reach the class
    int u_off, v_off;    // dY row / column of class pixel (0, 0) at tap (r0, t0)
    int block_begin;     // first block of the class
    int blocks;          // blocks of the class
    int ntiles;          // tiles of the class
    FastDiv fd_hw, fd_wc;
};

struct PArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, K, S, stride, Ho, Wo, Cg, Kg, G;
    int wk_stride;       // elements between W k-rows (R*S*Cg)
    int bm;              // valid pixels per tile (<= 224)
    int ctiles;          // Cg / 256
    int kchunks;         // 32-deep chunks of Kg (a multiple of 4)
    int nclasses;
    PClass cls[kPMaxClasses];
};

__device__ inline int p_swz_a(int row) { return (row >> 2) & 3; }
__device__ inline int p_swz_b(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }

// Pixel range of class tile lt: m in [m_lo, m_hi), group g, channels from c0.
struct PTile {
    int m_lo, m_hi, g, c0;
};

__device__ __attribute__((always_inline)) inline PTile p_tile(int lt, int ctiles, int G, int bm, int mc) {
    PTile t;
    const int ct = lt % ctiles, rest = lt / ctiles;
    t.g = rest % G;
    t.c0 = ct * kPBN;
    t.m_lo = (rest / G) * bm;
    t.m_hi = min(mc, t.m_lo + bm);
    return t;
}

template <typename T>
__global__ __launch_bounds__(kPThreads, 1) void dgrad_persist_kernel(const PArgs a) {
    constexpr int NM = kPWMB * kPWNB;           // MFMAs per wave per step
    __shared__ __attribute__((aligned(16))) unsigned char lds[kPLds + 8 * kPEpiWave];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = a.stride;
    const bool a2 = wave + 8 < kPARegs;         // this wave loads a second dY region

    // ---- block -> class (fixed for the block) and its range of tiles ----
    const int bid = blockIdx.x;
    int ci = 0;
#pragma unroll
    for (int i = 1; i < kPMaxClasses; ++i)
        if (i < a.nclasses && bid >= a.cls[i].block_begin) ci = i;
    const PClass cl = a.cls[ci];
    const int lb = bid - cl.block_begin;
    const int t_lo = int(int64_t(cl.ntiles) * lb / cl.blocks);
    const int t_hi = int(int64_t(cl.ntiles) * (lb + 1) / cl.blocks);
    const int hw = cl.hc * cl.wc;
    const int mc = a.N * hw;
    const int steps = cl.nr * cl.nt * a.kchunks;   // per tile, a multiple of 4

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // ---- per-lane load roles: dY region wave + 8*D (16 pixel rows), W region
    // wave + 8*E (2 k-rows) ----
    uint32_t b_voff[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int krow = 2 * (wave + 8 * e) + (lane >> 5);
        b_voff[e] = uint32_t((krow * a.wk_stride + ((lane & 31) ^ p_swz_b(krow)) * 8) * 2);
    }

    // ---- issue cursor: tile, tap (ti, tj), 32-deep chunk kk ----
    int i_t = t_lo, i_ti = 0, i_tj = 0, i_kk = 0;
    PTile it = p_tile(i_t, a.ctiles, a.G, a.bm, mc);
    uint32_t a_base[2];
    int a_u[2], a_v[2];
    // dY sources of tile i_t for this lane's rows: a_base = byte offset of the
    // row's pixel at tap (0, 0) plus its chunk, (a_u, a_v) that pixel; rows
    // past the tile (and all rows once the block's tiles are done) get
    // coordinates outside dY, so every tap reads zeros.
    auto set_tile = [&]() __attribute__((always_inline)) {
        it = p_tile(i_t, a.ctiles, a.G, a.bm, mc);
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const int row = 16 * (wave + 8 * d) + (lane >> 2);
            const int m = it.m_lo + row;
            a_base[d] = kOob;
            a_u[d] = a_v[d] = -(1 << 30);
            if (i_t < t_hi && row < a.bm && m < it.m_hi) {
                const int n = fdiv(m, cl.fd_hw);
                const int rem = m - n * hw;
                const int hc = fdiv(rem, cl.fd_wc);
                const int wc = rem - hc * cl.wc;
                const int u0 = hc + cl.u_off, v0 = wc + cl.v_off;
                a_u[d] = u0;
                a_v[d] = v0;
                a_base[d] = uint32_t((((n * a.Ho + u0) * a.Wo + v0) * a.K + it.g * a.Kg +
                                      ((lane & 3) ^ p_swz_a(row)) * 8) * 2);
            }
        }
        if (i_t >= t_hi) b_voff[0] = b_voff[1] = kOob;
    };
    set_tile();
    auto advance = [&]() __attribute__((always_inline)) {
        i_kk += kPBK;
        if (i_kk >= a.Kg) {
            i_kk = 0;
            if (++i_tj >= cl.nt) {
                i_tj = 0;
                if (++i_ti >= cl.nr) {
                    i_ti = 0;
                    ++i_t;
                    set_tile();
                }
            }
        }
    };
    // load X of the cursor's step into stage STG: 0, 1 dY regions, 2, 3 W regions
    auto load_one = [&](auto stg, auto xc) {
        constexpr int STG = decltype(stg)::value, X = decltype(xc)::value;
        (void)a_base; (void)a_u; (void)a_v; (void)b_voff;
        if constexpr (X < 2) {
            if (X == 1 && !a2) return;
            const uint32_t tap_bytes = uint32_t((i_ti * a.Wo + i_tj) * a.K * 2);
            const bool in = uint32_t(a_u[X] - i_ti) < uint32_t(a.Ho) &&
                            uint32_t(a_v[X] - i_tj) < uint32_t(a.Wo);
            dma16(rdy, lds + STG * kPABytes + (wave + 8 * X) * 1024, in ? a_base[X] - tap_bytes : kOob,
                  uint32_t(i_kk * 2));
        } else {
            constexpr int E = X - 2;
            const int rt = (cl.r0 + s * i_ti) * a.S + cl.t0 + s * i_tj;
            const uint32_t soff = uint32_t(((it.g * a.Kg + i_kk) * a.wk_stride + rt * a.Cg + it.c0) * 2);
            dma16(rw, lds + kPBBase + STG * kPBBytes + (wave + 8 * E) * 1024, b_voff[E], soff);
        }
    };
    // vmcnt(n * loads of this wave per step)
    auto wait_steps = [&](auto nc) {
        constexpr int N = decltype(nc)::value;
        if (a2) wait_vm<N * 4>();
        else wait_vm<N * 3>();
    };

    // ---- per-lane fragment addresses (stage 0; stages add an immediate) ----
    // dY fragment i of the wave sits 16 rows (1 KiB) after fragment i - 1 with
    // the same chunk swizzle (rows base + 16i + frow, (row >> 2) & 3 does not
    // depend on i), so one address serves all seven
    const int wm = wave >> 2, wn = wave & 3;
    const int frow = lane & 15, fgrp = lane >> 4;
    const uint32_t lds0 = lds_addr(lds);
    const uint32_t fa_addr = lds0 + (wm * (kPWMB * 16) + frow) * kPARow + ((fgrp ^ p_swz_a(frow)) << 4);
    // transpose read: the lane supplies k-row fgrp*8 + 4h + frow/4 at channel
    // .. + 4*(frow%4) and receives 4 consecutive k of one channel; the second
    // half (h = 1) is 4 rows (2 KiB) further with the same swizzle (h does not
    // touch bits 0, 1 and 3 of k)
    uint32_t fb_addr[kPWNB];
#pragma unroll
    for (int j = 0; j < kPWNB; ++j) {
        const int k = fgrp * 8 + (frow >> 2);
        const int c = wn * (kPWNB * 16) + j * 16 + 4 * (frow & 3);
        fb_addr[j] = lds0 + kPBBase + k * kPBRow + (((c >> 3) ^ p_swz_b(k)) << 4) + (c & 7) * 2;
    }

    f32x4 acc[kPWMB][kPWNB];
    // W fragments double-buffered (read a step ahead); each dY fragment is
    // re-read for the next step right after its last product of this one
    // (the matrix instruction has taken its A/B operands at issue)
    i32x4 fa[kPWMB];
    i32x2 fb[2][kPWNB][2];
    auto read_a = [&](auto stg, auto ic) {
        constexpr int STG = decltype(stg)::value, I = decltype(ic)::value;
        (void)fa; (void)fa_addr;
        // "+v": the fragment is rewritten in place (its product has issued)
        asm volatile("ds_read_b128 %0, %1 offset:%2"
                     : "+v"(fa[I])
                     : "v"(fa_addr), "i"(STG * kPABytes + I * 1024));
    };
    auto read_b = [&](auto stg, auto bc, auto rc) {
        constexpr int STG = decltype(stg)::value, B = decltype(bc)::value, R = decltype(rc)::value;
        (void)fb; (void)fb_addr;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(fb[B][R / 2][R % 2])
                     : "v"(fb_addr[R / 2]), "i"(STG * kPBBytes + (R % 2) * 4 * kPBRow));
    };
    // The reads are asm, invisible to the compiler's wait tracking: wait
    // explicitly and tie the fragments to the wait.  At the end of a step all
    // but the last kPTail dY reads (the newest LDS operations) must have
    // landed; those finish during the next step's first products and are
    // waited for before its first load (which overwrites their stage) and
    // before their own products.
    auto wait_frags = [&](auto bc, auto pending) {
        constexpr int B = decltype(bc)::value, P = decltype(pending)::value;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(fa[0]), "+v"(fb[B][0][0]) : "i"(P));
#pragma unroll
        for (int i = 1; i < kPWMB - P; ++i) asm volatile("" : "+v"(fa[i]));
#pragma unroll
        for (int j = 0; j < kPWNB; ++j) asm volatile("" : "+v"(fb[B][j][0]), "+v"(fb[B][j][1]));
    };
    auto wait_tail = [&](auto nc) {
        constexpr int N = decltype(nc)::value;   // LDS operations issued since
        (void)fa;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(fa[kPWMB - 2]), "+v"(fa[kPWMB - 1]) : "i"(N));
    };
    auto mfma_one = [&](auto bc, auto ic, auto jc) {
        constexpr int B = decltype(bc)::value, i = decltype(ic)::value, j = decltype(jc)::value;
        const i32x4 w4 = {fb[B][j][0][0], fb[B][j][0][1], fb[B][j][1][0], fb[B][j][1][1]};
        // transposed product: rows = channels (W), columns = pixels (dY)
        acc[i][j] = mfma16x16x32<T>(w4, fa[i], acc[i][j]);
    };

    // Byte offset of this lane's 128-byte dX slice (wave channels) for tile
    // row `row` of tile pt; kOob past the tile.
    auto px_off = [&](const PTile& pt, int row) __attribute__((always_inline)) -> uint32_t {
        const int m = pt.m_lo + row;
        if (row >= a.bm || m >= pt.m_hi) return kOob;
        const int n = fdiv(m, cl.fd_hw);
        const int rem = m - n * hw;
        const int hc = fdiv(rem, cl.fd_wc);
        const int wc = rem - hc * cl.wc;
        const int pix = (n * a.H + cl.a + s * hc) * a.W + cl.b + s * wc;
        return uint32_t((pix * a.C + pt.g * a.Cg + pt.c0 + wn * (kPWNB * 16)) * 2);
    };
    // Round and store pixel tile I of tile pt straight from the accumulators.
    // A lane holds 4 consecutive channels of one pixel per channel tile; the
    // row swap pairs lanes fgrp 2r and 2r+1 (16 lanes apart) so that, for two
    // adjacent channel tiles jp and jp+1, fgrp 0 ends with tile jp's channels
    // 0..7, fgrp 1 tile jp+1's 0..7, fgrp 2 and 3 the same for 8..15: the 4
    // lanes of a pixel write 64 contiguous bytes.
    auto store_rows = [&](auto ic, const PTile& pt) {
        constexpr int I = decltype(ic)::value;
        // lane-derived values recomputed here from a copy the compiler cannot
        // hoist out of the tile loop (they would otherwise stay live in
        // registers through every step)
        int l;
        asm volatile("v_mov_b32 %0, %1" : "=v"(l) : "v"(lane));
        const int lf = l & 15, lg = l >> 4;
        const uint32_t lane_off = uint32_t(((lg & 1) << 5) | ((lg >> 1) << 4));
        const uint32_t off = px_off(pt, wm * (kPWMB * 16) + I * 16 + lf) + lane_off;
#pragma unroll
        for (int jp = 0; jp < kPWNB; jp += 2) {
            const auto lo = __builtin_amdgcn_permlane16_swap(pack2<T>(acc[I][jp][0], acc[I][jp][1]),
                                                             pack2<T>(acc[I][jp + 1][0], acc[I][jp + 1][1]),
                                                             false, false);
            const auto hi = __builtin_amdgcn_permlane16_swap(pack2<T>(acc[I][jp][2], acc[I][jp][3]),
                                                             pack2<T>(acc[I][jp + 1][2], acc[I][jp + 1][3]),
                                                             false, false);
            const i32x4 v = {int(lo[0]), int(hi[0]), int(lo[1]), int(hi[1])};
            buf_store16(v, rdx, off + uint32_t(jp * 32));
        }
    };

    // One step out of stage STG (W fragments in buffer STG & 1, dY fragments
    // in fa, all read during the previous step).  The products of the first
    // kPPre pixel tiles need nothing new, so they issue before the wait for
    // the next stage and the barrier (every wave has also finished reading
    // this stage after it, so it takes the loads of the step three ahead):
    // the matrix cores stay busy while the slower wave of each SIMD reaches
    // the barrier.  The rest of the products follow pixel-tile by pixel-tile,
    // with the next step's W reads and the loads in the first gaps and each
    // dY fragment re-read after its last product.  The first step of a tile
    // (FIRST) stores the previous tile's sums from the accumulators before
    // anything else and starts its own products from zero.
    auto step = [&](auto stg, auto firstc, const PTile& prev) {
        constexpr int STG = decltype(stg)::value;
        constexpr bool FIRST = decltype(firstc)::value;
        constexpr int FB = STG & 1, NB = FB ^ 1, NXT = (STG + 1) % kPStages;
        if constexpr (FIRST) {
            sfor<kPWMB>([&](auto ic) {
                store_rows(ic, prev);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        auto product = [&](auto ic, auto jc) {
            constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
            if constexpr (FIRST) {
                const i32x4 w4 = {fb[FB][j][0][0], fb[FB][j][0][1], fb[FB][j][1][0], fb[FB][j][1][1]};
                acc[i][j] = mfma16x16x32<T>(w4, fa[i], f32x4{0.f, 0.f, 0.f, 0.f});
            } else {
                mfma_one(IC<FB>{}, ic, jc);
            }
        };
        sfor<kPPre * kPWNB>([&](auto mc) {
            constexpr int M = decltype(mc)::value;
            product(IC<M / kPWNB>{}, IC<M % kPWNB>{});
        });
        __builtin_amdgcn_sched_barrier(0);
        wait_steps(IC<kPStages - 2>{});
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        sfor<kPPre>([&](auto ic) { read_a(IC<NXT>{}, ic); });
        sfor<NM - kPPre * kPWNB>([&](auto mc) {
            constexpr int M = decltype(mc)::value + kPPre * kPWNB;
            constexpr int i = M / kPWNB, j = M % kPWNB;
            product(IC<i>{}, IC<j>{});
            if constexpr (j == kPWNB - 1) {
                read_a(IC<NXT>{}, IC<i>{});
            } else {
                constexpr int q = (i - kPPre) * (kPWNB - 1) + j;   // gap index
                if constexpr (q < 2 * kPWNB) {
                    read_b(IC<NXT>{}, IC<NB>{}, IC<q>{});
                } else if constexpr (q < 2 * kPWNB + 4) {
                    if constexpr (q == 2 * kPWNB) wait_tail(IC<p_lds_before_loads()>{});
                    load_one(stg, IC<q - 2 * kPWNB>{});
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        advance();
        wait_frags(IC<NB>{}, IC<kPTail>{});
    };

    // prologue: steps 0..3 into stages 0..3, then step 0's fragments
    sfor<kPStages>([&](auto sc) {
        sfor<4>([&](auto xc) { load_one(sc, xc); });
        advance();
    });
    wait_steps(IC<kPStages - 1>{});
    __builtin_amdgcn_s_barrier();
    sfor<kPWMB>([&](auto ic) { read_a(IC<0>{}, ic); });
    sfor<2 * kPWNB>([&](auto rc) { read_b(IC<0>{}, IC<0>{}, rc); });
    wait_frags(IC<0>{}, IC<0>{});

    // Tiles start at stage 0 (steps per tile are a multiple of 4).  The
    // previous tile of the first one is empty: its stores fall outside dX.
    PTile prev;
    prev.m_lo = prev.m_hi = 0;
    prev.g = prev.c0 = 0;
    using TrueT = std::true_type;
    using FalseT = std::false_type;
#pragma unroll 1
    for (int t = t_lo; t < t_hi; ++t) {
        step(IC<0>{}, TrueT{}, prev);
        step(IC<1>{}, FalseT{}, prev);
        step(IC<2>{}, FalseT{}, prev);
        step(IC<3>{}, FalseT{}, prev);
#pragma unroll 1
        for (int q = kPStages; q < steps; q += kPStages) {
            step(IC<0>{}, FalseT{}, prev);
            step(IC<1>{}, FalseT{}, prev);
            step(IC<2>{}, FalseT{}, prev);
            step(IC<3>{}, FalseT{}, prev);
        }
        prev = p_tile(t, a.ctiles, a.G, a.bm, mc);
    }
    wait_frags(IC<0>{}, IC<0>{});   // the last step's tail reads
    // The last tile: stored through the wave's own LDS staging area, 16
    // pixels at a time: the lanes write their 4-channel pieces (row = pixel,
    // 16-byte chunk index XOR-ed by row & 7), read back whole 128-byte rows
    // (8 lanes a row), and each store then writes 8 pixels' full 128-byte
    // slices (whole cache lines).  A wave's LDS accesses run in order, so no
    // barrier is needed.
    if (t_hi > t_lo) {
        unsigned char* epi = lds + kPLds + wave * kPEpiWave;
#pragma unroll
        for (int i = 0; i < kPWMB; ++i) {
#pragma unroll
            for (int j = 0; j < kPWNB; ++j) {
                const i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                                 int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
                const int chunk = (j * 2 + (fgrp >> 1)) ^ (frow & 7);
                *reinterpret_cast<i32x2*>(epi + frow * 128 + chunk * 16 + (fgrp & 1) * 8) = v;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = (lane >> 3) + 8 * h;
                const i32x4 v = *reinterpret_cast<const i32x4*>(epi + r * 128 + (((lane & 7) ^ (r & 7)) << 4));
                buf_store16(v, rdx, px_off(prev, wm * (kPWMB * 16) + i * 16 + r) + uint32_t((lane & 7) * 16));
            }
        }
    }
    wait_vm<0>();   // loads issued past the last step still target LDS
}

struct HClass {
    PClass c;
    int64_t mc;     // class pixels
    int steps;      // reduction steps per tile
};

}  // namespace

std::string dgrad_persist_reason(const Prob& p) {
    if (p.cg % kPBN != 0) return "persistent strided dgrad needs channels per group of dx a multiple of 256";
    if (p.kg % (kPStages * kPBK) != 0)
        return "persistent strided dgrad needs channels per group of dy a multiple of 128";
    if (p.stride > 4) return "persistent strided dgrad supports stride <= 4";
    if (p.stride > p.r || p.stride > p.s)
        return "persistent strided dgrad needs stride <= R and <= S (every phase class has a tap)";
    return "";
}

bool dgrad_persist_taken(const Prob& p, const Plan& pl) {
    if (pl.variant != CNHWC_VAR_DGRAD_IGEMM) return false;
    if (!(pl.tune == 5 || (pl.tune == 0 && p.stride >= 2))) return false;
    return dgrad_persist_reason(p).empty();
}

int launch_dgrad_persist(const Prob& p, const void* dy, const void* w, void* dx, hipStream_t st) {
    if (!dgrad_persist_reason(p).empty()) return CNHWC_UNSUPPORTED;
    PArgs a{};
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.S = int(p.s); a.stride = p.stride;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg); a.G = p.groups;
    a.wk_stride = int(p.r * p.s * p.cg);
    a.ctiles = int(p.cg / kPBN);
    a.kchunks = int(p.kg / kPBK);
    const int s = p.stride;
    HClass tmp[kPMaxClasses];
    int nc = 0;
    for (int ca = 0; ca < s; ++ca)
        for (int cb = 0; cb < s; ++cb) {
            PClass c{};
            c.a = ca; c.b = cb;
            c.hc = int((p.h - ca + s - 1) / s);
            c.wc = int((p.w - cb + s - 1) / s);
            if (c.hc <= 0 || c.wc <= 0) continue;
            c.r0 = (ca + p.pad_h) % s;
            c.t0 = (cb + p.pad_w) % s;
            c.nr = int((p.r - c.r0 + s - 1) / s);   // >= 1: stride <= R, S
            c.nt = int((p.s - c.t0 + s - 1) / s);
            c.u_off = (ca + p.pad_h - c.r0) / s;
            c.v_off = (cb + p.pad_w - c.t0) / s;
            c.fd_hw = make_fastdiv(uint32_t(c.hc * c.wc));
            c.fd_wc = make_fastdiv(uint32_t(c.wc));
            tmp[nc++] = HClass{c, p.n * c.hc * c.wc, c.nr * c.nt * a.kchunks};
        }
    if (nc == 0) return CNHWC_OK;
    // heaviest class first (its blocks are dispatched first)
    std::stable_sort(tmp, tmp + nc, [](const HClass& x, const HClass& y) { return x.steps > y.steps; });
    // tile height: the full 224 pixels unless the problem has fewer tiles
    // than CUs, then shorter tiles (down to half) for more of them
    const int64_t per_m = int64_t(a.ctiles) * a.G;
    auto count_tiles = [&](int bm) {
        int64_t t = 0;
        for (int i = 0; i < nc; ++i) t += (tmp[i].mc + bm - 1) / bm * per_m;
        return t;
    };
    int bm = kPBM;
    while (bm > kPBM / 2 && count_tiles(bm) < kNumCUs) bm -= 16;
    a.bm = bm;
    // blocks per class: one each, then each further CU to the class whose
    // blocks run the most steps (ceil(tiles / blocks) * steps per tile)
    int64_t nt[kPMaxClasses], nb[kPMaxClasses];
    int used = 0;
    for (int i = 0; i < nc; ++i) {
        nt[i] = (tmp[i].mc + bm - 1) / bm * per_m;
        nb[i] = 1;
        ++used;
    }
    for (; used < kNumCUs; ++used) {
        int best = -1;
        int64_t best_len = 0;
        for (int i = 0; i < nc; ++i) {
            if (nb[i] >= nt[i]) continue;
            const int64_t len = (nt[i] + nb[i] - 1) / nb[i] * tmp[i].steps;
            if (len > best_len) { best_len = len; best = i; }
        }
        if (best < 0) break;
        ++nb[best];
    }
    if (used > kNumCUs) return CNHWC_UNSUPPORTED;   // more classes than CUs (stride <= 4: at most 16)
    int grid = 0;
    for (int i = 0; i < nc; ++i) {
        PClass& c = tmp[i].c;
        c.ntiles = int(nt[i]);
        c.blocks = int(nb[i]);
        c.block_begin = grid;
        grid += c.blocks;
        a.cls[i] = c;
    }
    a.nclasses = nc;
    if (p.dtype == CNHWC_BF16)
        hipLaunchKernelGGL((dgrad_persist_kernel<BF16>), dim3(grid), dim3(kPThreads), 0, st, a);
    else
        hipLaunchKernelGGL((dgrad_persist_kernel<F16>), dim3(grid), dim3(kPThreads), 0, st, a);
    return CNHWC_OK;
}

}  // namespace cnhwc
