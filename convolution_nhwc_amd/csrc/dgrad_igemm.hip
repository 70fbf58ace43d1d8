// Backward-data convolution as implicit GEMMs on the gfx950 matrix cores:
// a ring kernel (both operands streamed per reduction step; also the 1x1
// pointwise fast path, as a compile-time specialisation), a dY-window kernel
// for stride-1 problems whose filters have two or more taps, and two
// pointwise kernels for narrow dX (C <= 64) that keep the filter on chip: a
// row-streamed one (K = 64..256 in steps of 64) and an LDS-persistent one.
// All pointwise paths produce the same bits as the general ring kernel.
//
// Strided dgrad splits dX into stride*stride phase classes (h mod s, w mod s)
// -- the "tilde" decomposition of "perf(rocke/conv): add the pointwise fast
// path dgrad was missing" (Finding 4 and the fast-path commit).  In class
// (a, b) only the filter rows r = (a + pad_h) mod s + s*i and columns
// t = (b + pad_w) mod s + s*j touch dX, and dY row (h + pad_h - r)/s moves by
// exactly one row per step of i, so each class is a dense GEMM
//     dX_class[m, c] = sum_{i, j, k} dY[n, u0(m) - i, v0(m) - j, g*Kg + k] * W[g*Kg + k, r_i, t_j, c]
// with M = the class's pixels, N = Cg, and reduction Kg * taps.  Classes with
// no tap write zeros.  All classes of a kernel run in one launch, heaviest
// first; a block finds its class in a small table in the kernel arguments (a
// few scalar compares, no divide in the reduction loop).
//
// For 1x1, stride 1, no padding and one group the decomposition is the
// identity (one class, Hc = H, Wc = W, one tap): the dY offset of GEMM row m is
// m*K + k and the W offset is k*C + c (same page, the fast-path commit).  The PW
// specialisation uses exactly those offsets; the reduction order (ascending
// 32-deep MFMA steps with the same lane/k assignment) and the rounding are the
// same, so it is bit-identical to the general kernel on the same problem (the
// general path runs one-tap classes on this same ring kernel).
//
// Ring kernel data path (gfx950): both operands go global -> LDS with
// asynchronous buffer loads that write LDS directly (no VGPR staging) into a
// ring of three stages, so two 64-deep reduction steps are in flight while one
// is multiplied.  dY tiles are 128-byte k-rows (16-byte chunks XOR-swizzled by
// row); W tiles keep their natural c-contiguous rows (chunks swizzled by k) and
// are read as MFMA operands with the LDS transpose read (ds_read_b64_tr_b16),
// which hands each lane four consecutive k of one channel.  Per-lane base
// addresses are computed once; in the loop the uniform parts of the global
// offsets go in the scalar offset field, the stage offsets in the LDS
// instructions' immediate field, and a tap is valid for a row when the row's
// dY coordinates minus the tap's offsets fall inside dY (else the load offset
// is out of range, so the buffer descriptor returns zeros).  Each step's LDS
// reads and loads are
// placed between its matrix instructions.  The MFMA computes the transposed
// tile (channels x pixels) so each lane ends with four consecutive channels of
// one pixel; the epilogue rounds to fp16/bf16 (RNE) and restages through LDS
// for full 16-byte row stores.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>
#include <type_traits>
#include <utility>

namespace cnhwc {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;          // reduction depth per stage (elements)
constexpr int kARow = 128;       // bytes per dY row of a stage
constexpr int kStages = 3;
constexpr int kMaxClasses = 16;

struct ClassInfo {
    int a, b;          // phase of the class: h = a + s*hc, w = b + s*wc
    int hc, wc;        // rows / columns of dX in the class
    int r0, t0;        // first filter row / column touching the class
    int nr, nt;        // number of such rows / columns
    int tile_begin;    // first block of the class
    int mtiles;        // M tiles of the class
    int u_off, v_off;  // dY row / column of class pixel (0, 0) at tap (r0, t0)
    FastDiv fd_hw, fd_wc;  // division by hc * wc and by wc (pixel -> n, row, column)
};

struct IgemmArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, K, R, S, stride, pad_h, pad_w, Ho, Wo, Cg, Kg, G;
    int bm;            // valid pixels per M tile (<= the tile's capacity)
    int ctiles;        // ceil(Cg / BN)
    int nclasses;
    int remap;         // 1: remap block ids so each XCD works on contiguous tiles
    int splits;        // split-K: reduction splits (grid y); 1 otherwise
    float* ws;         // split-K: fp32 partials [split][N*H*W][C]
    ClassInfo cls[kMaxClasses];
};



// Chunk swizzles.  dY rows (128 B): 16-byte chunk ^ f(row) so that the 16
// rows one fragment read touches hit distinct bank groups.  W rows: the
// transpose read of a 16-lane group touches k-rows k0..k0+3 (and k0+8.. in the
// neighbouring group) two chunks apiece; XOR-ing the chunk pair index with a
// different value per row keeps those rows' chunk pairs apart.
__device__ inline int swz_a(int row) { return (row ^ (row >> 3)) & 7; }
template <int CHUNKS>
__device__ inline int swz_b(int k) {
    if constexpr (CHUNKS == 16) return 2 * ((k & 3) | ((k >> 1) & 4));
    else return 2 * (((k >> 1) & 1) | ((k >> 2) & 2));
}


template <typename T, int WMB, int WNB, bool PW, bool KR, bool SK>
__global__ __launch_bounds__(kThreads, 1) void dgrad_igemm_kernel(const IgemmArgs a) {
    constexpr int WAVES_M = 2, WAVES_N = 2;
    constexpr int BMC = WAVES_M * WMB * 16;             // tile capacity in pixels
    constexpr int BN = WAVES_N * WNB * 16;              // channels per tile
    constexpr int A_BYTES = BMC * kARow;                // one A stage
    constexpr int B_ROW = BN * 2;                       // bytes of one W k-row
    constexpr int B_CHUNKS = BN / 8;                    // 16-byte chunks per W row
    constexpr int B_BYTES = kBK * B_ROW;                // one B stage
    constexpr int B_BASE = kStages * A_BYTES;           // B stages follow the A stages
    constexpr int A_REG = A_BYTES / 1024 / 4;           // 1 KiB A regions per wave
    constexpr int B_REG = B_BYTES / 1024 / 4;           // 1 KiB B regions per wave
    constexpr int B_ROWS_PER_REG = 1024 / B_ROW;
    constexpr int LOADS = A_REG + B_REG;                // async loads per lane per stage
    constexpr int C_STRIDE = BN * 2 + 16;
    static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "regions split over 4 waves");
    static_assert(B_CHUNKS == 8 || B_CHUNKS == 16, "W row swizzle");
    static_assert(BMC * C_STRIDE <= kStages * (A_BYTES + B_BYTES), "epilogue tile fits");
    static_assert((kStages - 1) * A_BYTES < 65536 && (kStages - 1) * B_BYTES < 65536,
                  "stage offsets fit the LDS immediate");
    static_assert(LOADS * (kStages - 1) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) unsigned char lds[kStages * (A_BYTES + B_BYTES)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS pointers scalar

    // ---- block -> (class, m tile, group, c tile) ----
    const int bid = blockIdx.x;
    int ci = 0;
    // every class's first block is read at once (constant indices: the
    // scalar loads issue together and one wait covers them)
#pragma unroll
    for (int i = 1; i < kMaxClasses; ++i)
        if (i < a.nclasses && bid >= a.cls[i].tile_begin) ci = i;
    const ClassInfo cl = a.cls[ci];
    int local = bid - cl.tile_begin;
    if (a.remap) {
        // blocks go to the 8 XCDs round-robin; give each XCD a contiguous run
        // of tiles so neighbouring tiles share that XCD's L2
        const int cnt = cl.mtiles * a.ctiles * a.G;
        local = (local & 7) * (cnt >> 3) + (local >> 3);
    }
    const int ct = local % a.ctiles;
    const int rest = local / a.ctiles;
    const int g = rest % a.G;
    const int mt = rest / a.G;
    const int c0 = ct * BN;
    const int Mc = a.N * cl.hc * cl.wc;
    const int s = a.stride;
    const int m_lo = mt * a.bm;
    const int m_hi = min(Mc, m_lo + a.bm);

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // ---- per-lane A (dY) sources: region q = wave + 4*i holds rows 8q .. 8q+7 ----
    // a_base: byte offset of the row's dY pixel at tap (0, 0) plus its chunk
    // (kOob past the tile); (a_u, a_v): that pixel's dY row and column.  Tap
    // (ti, tj) of the class reads dY pixel (a_u - ti, a_v - tj): the load
    // offset is (a_base - tap_bytes), replaced by an out-of-range offset
    // (a zero read through the buffer range check) when that pixel is outside
    // dY.  Rows past the tile get a_u = a_v = -2^30, outside for every tap.
    uint32_t a_base[A_REG];
    int a_u[A_REG], a_v[A_REG];
    int a_kq[A_REG];
#pragma unroll
    for (int i = 0; i < A_REG; ++i) {
        const int row = 8 * (wave + 4 * i) + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_a(row);
        a_kq[i] = chunk * 8;
        const int m = m_lo + row;
        a_base[i] = kOob;
        a_u[i] = a_v[i] = -(1 << 30);
        if (row < a.bm && m < m_hi) {
            if (PW) {
                a_base[i] = uint32_t((m * a.K + g * a.Kg + chunk * 8) * 2);
            } else {
                const int hw = cl.hc * cl.wc;
                const int n = fdiv(m, cl.fd_hw);
                const int rem = m - n * hw;
                const int hc = fdiv(rem, cl.fd_wc);
                const int wc = rem - hc * cl.wc;
                const int u0 = hc + cl.u_off;
                const int v0 = wc + cl.v_off;
                a_u[i] = u0;
                a_v[i] = v0;
                a_base[i] = uint32_t((((n * a.Ho + u0) * a.Wo + v0) * a.K + g * a.Kg + chunk * 8) * 2);
            }
        }
    }
    // ---- per-lane B (W) sources: region q = wave + 4*i holds k-rows B_ROWS_PER_REG*q .. ----
    const int taps_rs = PW ? 1 : a.R * a.S;
    const int wk_stride = taps_rs * a.Cg;                // elements between W k-rows
    uint32_t b_voff[B_REG];
    int b_krow[B_REG];
#pragma unroll
    for (int i = 0; i < B_REG; ++i) {
        const int q = wave + 4 * i;
        const int krow = B_ROWS_PER_REG * q + lane / B_CHUNKS;
        const int chunk = (lane % B_CHUNKS) ^ swz_b<B_CHUNKS>(krow);
        const int c = c0 + chunk * 8;
        b_krow[i] = krow;
        b_voff[i] = c < a.Cg ? uint32_t((krow * wk_stride + chunk * 8) * 2) : kOob;
    }

    const int kchunks = (a.Kg + kBK - 1) / kBK;
    int steps = cl.nr * cl.nt * kchunks;
    int step0 = 0;
    if constexpr (SK) {
        // split-K: this block takes reduction steps [step0, step0 + steps) of
        // the tile (contiguous, balanced; empty when splits exceed the steps)
        const int split = blockIdx.y;
        step0 = int(int64_t(steps) * split / a.splits);
        steps = int(int64_t(steps) * (split + 1) / a.splits) - step0;
    }

    // Issue cursor (uniform): reduction step = (tap (ti, tj), 64-deep chunk kk).
    // It runs two steps ahead of the multiply and is advanced without
    // branches; past the last step it keeps producing offsets whose loads are
    // either range-checked zeros or in-range data of stages never multiplied.
    const int tap0 = step0 / kchunks;
    int cur_kk = (step0 - tap0 * kchunks) * kBK;
    int cur_ti = cl.nt > 0 ? tap0 / cl.nt : 0;
    int cur_tj = tap0 - cur_ti * cl.nt;
    auto advance = [&]() {
        cur_kk += kBK;
        const bool wrap = cur_kk >= a.Kg;
        cur_kk = wrap ? 0 : cur_kk;
        cur_tj += wrap ? 1 : 0;
        const bool wrap2 = cur_tj >= cl.nt;
        cur_tj = wrap2 ? 0 : cur_tj;
        cur_ti += wrap2 ? 1 : 0;
    };
    // one async 16-byte load per lane into region D of stage STG (D < A_REG:
    // dY rows, else W k-rows)
    auto dma_one = [&](auto stg, auto dsc) {
        constexpr int STG = decltype(stg)::value, D = decltype(dsc)::value;
        (void)a_base; (void)a_u; (void)a_v; (void)a_kq; (void)b_voff; (void)b_krow;
        if constexpr (D < A_REG) {
            uint32_t v = a_base[D];
            if constexpr (!PW) {
                const uint32_t tap_bytes = uint32_t((cur_ti * a.Wo + cur_tj) * a.K * 2);
                const bool in = uint32_t(a_u[D] - cur_ti) < uint32_t(a.Ho) &&
                                uint32_t(a_v[D] - cur_tj) < uint32_t(a.Wo);
                v = in ? v - tap_bytes : kOob;
            }
            if (KR) v = (cur_kk + a_kq[D] < a.Kg) ? v : kOob;
            dma16(rdy, lds + STG * A_BYTES + (wave + 4 * D) * 1024, v, uint32_t(cur_kk * 2));
        } else {
            constexpr int E = D - A_REG;
            const int rt = PW ? 0 : (cl.r0 + s * cur_ti) * a.S + cl.t0 + s * cur_tj;
            const uint32_t b_soff = uint32_t(((g * a.Kg + cur_kk) * wk_stride + rt * a.Cg + c0) * 2);
            uint32_t v = b_voff[E];
            if (KR) v = (cur_kk + b_krow[E] < a.Kg) ? v : kOob;
            dma16(rw, lds + B_BASE + STG * B_BYTES + (wave + 4 * E) * 1024, v, b_soff);
        }
    };

    // ---- per-lane LDS fragment addresses (stage 0; stages add an immediate) ----
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int frow = lane & 15, fgrp = lane >> 4;
    uint32_t fa_addr[2][WMB];
    uint32_t fb_addr[2][WNB][2];
    const uint32_t lds0 = lds_addr(lds);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int chunk = ks * 4 + fgrp;
#pragma unroll
        for (int i = 0; i < WMB; ++i) {
            const int row = wm * (WMB * 16) + i * 16 + frow;
            fa_addr[ks][i] = lds0 + row * kARow + ((chunk ^ swz_a(row)) << 4);
        }
#pragma unroll
        for (int j = 0; j < WNB; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // transpose read: lane supplies k-row (.. + frow/4) at channel (.. + 4*(frow%4))
                const int k = ks * 32 + fgrp * 8 + 4 * h + (frow >> 2);
                const int c = wn * (WNB * 16) + j * 16 + 4 * (frow & 3);
                fb_addr[ks][j][h] = lds0 + B_BASE + k * B_ROW +
                                    (((c >> 3) ^ swz_b<B_CHUNKS>(k)) << 4) + (c & 7) * 2;
            }
    }

    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragments: [half of the 64-deep step][tile]; W tiles as two 8-byte halves
    i32x4 fa[2][WMB];
    i32x2 fb[2][WNB][2];
    constexpr int NREAD = 2 * WNB + WMB;   // LDS reads per half step
    // read R of half KS out of stage STG (R < 2*WNB: W transpose reads)
    auto read_one = [&](auto stg, auto ksc, auto rc) {
        constexpr int STG = decltype(stg)::value, KS = decltype(ksc)::value;
        constexpr int R = decltype(rc)::value;
        (void)fa; (void)fb; (void)fa_addr; (void)fb_addr;   // captured for every instantiation
        if constexpr (R < 2 * WNB) {
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(fb[KS][R / 2][R % 2])
                         : "v"(fb_addr[KS][R / 2][R % 2]), "i"(STG * B_BYTES));
        } else {
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(fa[KS][R - 2 * WNB])
                         : "v"(fa_addr[KS][R - 2 * WNB]), "i"(STG * A_BYTES));
        }
    };
    // the LDS reads are issued in asm, invisible to the compiler's wait
    // tracking: wait here and tie the fragments to the wait
    auto wait_frags = [&](auto ksc) {
        constexpr int KS = decltype(ksc)::value;
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[KS][0]), "+v"(fb[KS][0][0]));
#pragma unroll
        for (int i = 1; i < WMB; ++i) asm volatile("" : "+v"(fa[KS][i]));
#pragma unroll
        for (int j = 0; j < WNB; ++j) asm volatile("" : "+v"(fb[KS][j][0]), "+v"(fb[KS][j][1]));
    };
    auto mfma_one = [&](auto ksc, auto mc) {
        constexpr int KS = decltype(ksc)::value, M = decltype(mc)::value;
        constexpr int i = M / WNB, j = M % WNB;
        const i32x4 b = {fb[KS][j][0][0], fb[KS][j][0][1], fb[KS][j][1][0], fb[KS][j][1][1]};
        // transposed product: rows = channels (W), columns = pixels (dY)
        acc[i][j] = mfma16x16x32<T>(b, fa[KS][i], acc[i][j]);
    };

    // One reduction step out of stage STG, in two halves of 32.  First half:
    // multiply half 0 while reading half 1's fragments and issuing the loads
    // of the step two ahead into the stage freed by the previous step.  Then
    // wait for the next stage to land (own loads + barrier).  Second half:
    // multiply half 1 while reading half 0 of the next step.  Every LDS read
    // and load is placed between two matrix instructions (scheduling
    // barriers keep the order), so they issue under the matrix cores' work.
    constexpr int NM = WMB * WNB;
    constexpr int NI0 = NREAD + LOADS;
    constexpr int PER0 = (NI0 + NM - 1) / NM;
    constexpr int PER1 = (NREAD + NM - 1) / NM;
    auto step_fn = [&](auto stg) {
        constexpr int STG = decltype(stg)::value;
        constexpr int NXT = (STG + 1) % kStages, FREE = (STG + kStages - 1) % kStages;
        sfor<NM>([&](auto mc) {
            constexpr int M = decltype(mc)::value;
            mfma_one(IC<0>{}, mc);
            sfor<PER0>([&](auto pc) {
                constexpr int X = M * PER0 + decltype(pc)::value;
                if constexpr (X < NREAD) read_one(stg, IC<1>{}, IC<X>{});
                else if constexpr (X < NI0) dma_one(IC<FREE>{}, IC<X - NREAD>{});
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        advance();
        wait_frags(IC<1>{});
        wait_vm<LOADS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        sfor<NM>([&](auto mc) {
            constexpr int M = decltype(mc)::value;
            mfma_one(IC<1>{}, mc);
            sfor<PER1>([&](auto pc) {
                constexpr int X = M * PER1 + decltype(pc)::value;
                if constexpr (X < NREAD) read_one(IC<NXT>{}, IC<0>{}, IC<X>{});
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        wait_frags(IC<0>{});
    };

    if (steps > 0) {
        sfor<LOADS>([&](auto dc) { dma_one(IC<0>{}, dc); });
        advance();
        sfor<LOADS>([&](auto dc) { dma_one(IC<1>{}, dc); });
        advance();
        wait_vm<LOADS>();
        __builtin_amdgcn_s_barrier();
        sfor<NREAD>([&](auto rc) { read_one(IC<0>{}, IC<0>{}, rc); });
        wait_frags(IC<0>{});
#pragma unroll 1
        for (int st = 0; st < steps; st += kStages) {
            step_fn(IC<0>{});
            if (st + 1 < steps) step_fn(IC<1>{});
            if (st + 2 < steps) step_fn(IC<2>{});
        }
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
    }

    if constexpr (SK) {
        // ---- split-K epilogue: the fp32 partial tile straight to the
        // workspace, each lane's 4 consecutive channels as one 16-byte store;
        // every position of the tile is written (zeros for an empty split) ----
        float* wsp = a.ws + int64_t(blockIdx.y) * (int64_t(a.N) * a.H * a.W * a.C);
#pragma unroll
        for (int i = 0; i < WMB; ++i) {
            const int row = wm * (WMB * 16) + i * 16 + frow;
            const int m = m_lo + row;
            if (row >= a.bm || m >= m_hi) continue;
            const int hw = cl.hc * cl.wc;
            const int n = fdiv(m, cl.fd_hw);
            const int rem = m - n * hw;
            const int hc = fdiv(rem, cl.fd_wc);
            const int wc = rem - hc * cl.wc;
            const int64_t pix = (int64_t(n) * a.H + cl.a + s * hc) * a.W + cl.b + s * wc;
#pragma unroll
            for (int j = 0; j < WNB; ++j) {
                const int c = c0 + wn * (WNB * 16) + j * 16 + fgrp * 4;
                if (c < a.Cg)
                    *reinterpret_cast<f32x4*>(wsp + pix * a.C + g * a.Cg + c) = acc[i][j];
            }
        }
        return;
    }
    // ---- epilogue: round, stage the tile in LDS, 16-byte row stores ----
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j) {
            const int row = wm * (WMB * 16) + i * 16 + frow;     // pixel
            const int col = wn * (WNB * 16) + j * 16 + fgrp * 4; // first of 4 channels
            i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                       int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
            *reinterpret_cast<i32x2*>(lds + row * C_STRIDE + col * 2) = v;
        }
    __syncthreads();
    constexpr int CPR = BN / 8;  // 16-byte chunks per row
    for (int q = tid; q < BMC * CPR; q += kThreads) {
        const int row = q / CPR, cc = q % CPR;
        const int m = m_lo + row;
        const int c = c0 + cc * 8;
        if (row >= a.bm || m >= m_hi || c >= a.Cg) continue;
        int pix;
        if (PW) {
            pix = m;
        } else {
            const int hw = cl.hc * cl.wc;
            const int n = fdiv(m, cl.fd_hw);
            const int rem = m - n * hw;
            const int hc = fdiv(rem, cl.fd_wc);
            const int wc = rem - hc * cl.wc;
            pix = (n * a.H + cl.a + s * hc) * a.W + cl.b + s * wc;
        }
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + row * C_STRIDE + cc * 16);
        buf_store16(v, rdx, uint32_t(pix * a.C + g * a.Cg + c) * 2u);
    }
}

// ---------------------------------------------------------------------------
// Pointwise (1x1) dgrad for C <= 64: persistent, filter resident in LDS.
//
// The operands and the per-output reduction are those of the ring kernel's
// pointwise specialisation with its 128 x 64 tile (same fragments, same
// ascending 32-deep MFMA chain per output, same rounding), so the results are
// bit-identical.  What changes is the schedule around them:
//   * the whole filter (K x 64 channels, 128-byte k-rows swizzled like a W
//     stage) is loaded into LDS once per block, so the ring carries dY only;
//   * one block per CU walks M tiles b, b + G, b + 2G, ... and all their
//     64-deep reduction steps flow through one ring of NS dY stages, so up to
//     NS - 1 steps of dY loads stay in flight across tile boundaries;
//   * a finished tile is rounded into the dY stage it has just consumed (no
//     other loads target that stage until the next step) and written back as
//     full 128-byte pixel rows while the next tile's loads are in flight.
struct PwArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int M, C, K;       // pixels, channels of dX (<= 64), channels of dY
    int kpad;          // K rounded up to the 64-deep step
    int bm;            // pixels per tile (<= 128)
    int ntiles;        // M tiles
    int nblocks;       // grid size G (<= ntiles)
};

constexpr int kPwBM = 128;                  // tile capacity: 2 waves x 4 x 16 pixels
constexpr int kPwBN = 64;                   // channels: 2 waves x 2 x 16
constexpr int kPwStage = kPwBM * kARow;     // one 64-deep dY stage (16 KiB)
constexpr int kPwLds = 160 * 1024;          // LDS per CU

template <typename T, int NS, bool KR>
__global__ __launch_bounds__(kThreads, 1) void dgrad_pw_persist_kernel(const PwArgs a) {
    constexpr int WMB = 4, WNB = 2, WAVES_N = 2;
    constexpr int A_BYTES = kPwStage;
    constexpr int B_ROW = kPwBN * 2;                 // bytes of one filter k-row
    constexpr int LOADS = A_BYTES / 1024 / 4;        // async loads per lane per stage
    constexpr int W_BASE = NS * A_BYTES;             // the filter follows the stages
    constexpr int NLOW = NS < 4 ? NS : 4;            // stages addressed off the first base
    static_assert(LOADS * NS < 64, "vmcnt range");
    static_assert((NLOW - 1) * A_BYTES < 65536, "stage offsets fit the LDS immediate");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int G = a.nblocks;
    const int my_tiles = (a.ntiles - b + G - 1) / G;
    const int steps = my_tiles * (a.kpad / kBK);

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // ---- filter -> LDS once: 1 KiB regions of 8 k-rows, rows past K and
    // channels past C read as zeros ----
#pragma unroll 1
    for (int q = wave; q < a.kpad / 8; q += 4) {
        const int row = 8 * q + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_b<8>(row);
        const uint32_t v = (row < a.K && chunk * 8 < a.C) ? uint32_t((row * a.C + chunk * 8) * 2) : kOob;
        dma16(rw, lds + W_BASE + q * 1024, v, 0);
    }

    // ---- per-lane dY sources (tile-relative): region q = wave + 4*i holds rows 8q .. 8q+7 ----
    uint32_t a_off[LOADS];
    int a_row[LOADS], a_kq[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int row = 8 * (wave + 4 * i) + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_a(row);
        a_row[i] = row;
        a_kq[i] = chunk * 8;
        a_off[i] = uint32_t((row * a.K + chunk * 8) * 2);
    }
    // issue cursor (uniform): tile and 64-deep chunk of the step being loaded
    int i_mt = b, i_kk = 0;
    int i_lim = min(a.bm, a.M - i_mt * a.bm);        // valid rows of the tile
    auto advance_i = [&]() {
        i_kk += kBK;
        if (i_kk >= a.kpad) {
            i_kk = 0;
            i_mt += G;
            i_lim = min(a.bm, a.M - i_mt * a.bm);
        }
    };
    auto dma_one = [&](auto stg, auto dsc) {
        constexpr int STG = decltype(stg)::value, D = decltype(dsc)::value;
        (void)a_off; (void)a_row; (void)a_kq;
        uint32_t v = a_row[D] < i_lim ? a_off[D] : kOob;
        if (KR) v = (i_kk + a_kq[D] < a.K) ? v : kOob;
        dma16(rdy, lds + STG * A_BYTES + (wave + 4 * D) * 1024, v,
              uint32_t((i_mt * a.bm * a.K + i_kk) * 2));
    };

    // ---- per-lane LDS fragment addresses ----
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int frow = lane & 15, fgrp = lane >> 4;
    uint32_t fa_addr[2][WMB];     // stage 0 (stages 1..NLOW-1 add an immediate)
    uint32_t fa_hi[2][WMB];       // stage NLOW (stages above add an immediate)
    uint32_t fb_addr[2][WNB][2];  // filter k-rows 0..63 (a step adds its chunk offset)
    const uint32_t lds0 = lds_addr(lds);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int chunk = ks * 4 + fgrp;
#pragma unroll
        for (int i = 0; i < WMB; ++i) {
            const int row = wm * (WMB * 16) + i * 16 + frow;
            fa_addr[ks][i] = lds0 + row * kARow + ((chunk ^ swz_a(row)) << 4);
            fa_hi[ks][i] = fa_addr[ks][i] + NLOW * A_BYTES;
        }
#pragma unroll
        for (int j = 0; j < WNB; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = ks * 32 + fgrp * 8 + 4 * h + (frow >> 2);
                const int c = wn * (WNB * 16) + j * 16 + 4 * (frow & 3);
                fb_addr[ks][j][h] = lds0 + W_BASE + k * B_ROW +
                                    (((c >> 3) ^ swz_b<8>(k)) << 4) + (c & 7) * 2;
            }
    }

    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 fa[2][WMB];
    i32x2 fb[2][WNB][2];
    constexpr int NREAD = 2 * WNB + WMB;
    // read R of half KS: filter rows at byte offset wofs, dY out of stage STG
    auto read_one = [&](auto stg, auto ksc, auto rc, uint32_t wofs) {
        constexpr int STG = decltype(stg)::value, KS = decltype(ksc)::value;
        constexpr int R = decltype(rc)::value;
        (void)fa; (void)fb; (void)fa_addr; (void)fa_hi; (void)fb_addr;
        if constexpr (R < 2 * WNB) {
            asm volatile("ds_read_b64_tr_b16 %0, %1"
                         : "=v"(fb[KS][R / 2][R % 2])
                         : "v"(fb_addr[KS][R / 2][R % 2] + wofs));
        } else if constexpr (STG < NLOW) {
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(fa[KS][R - 2 * WNB])
                         : "v"(fa_addr[KS][R - 2 * WNB]), "i"(STG * A_BYTES));
        } else {
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(fa[KS][R - 2 * WNB])
                         : "v"(fa_hi[KS][R - 2 * WNB]), "i"((STG - NLOW) * A_BYTES));
        }
    };
    auto wait_frags = [&](auto ksc) {
        constexpr int KS = decltype(ksc)::value;
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[KS][0]), "+v"(fb[KS][0][0]));
#pragma unroll
        for (int i = 1; i < WMB; ++i) asm volatile("" : "+v"(fa[KS][i]));
#pragma unroll
        for (int j = 0; j < WNB; ++j) asm volatile("" : "+v"(fb[KS][j][0]), "+v"(fb[KS][j][1]));
    };
    auto mfma_one = [&](auto ksc, auto mc) {
        constexpr int KS = decltype(ksc)::value, M = decltype(mc)::value;
        constexpr int i = M / WNB, j = M % WNB;
        const i32x4 bb = {fb[KS][j][0][0], fb[KS][j][0][1], fb[KS][j][1][0], fb[KS][j][1][1]};
        acc[i][j] = mfma16x16x32<T>(bb, fa[KS][i], acc[i][j]);
    };

    // tile being multiplied and its reduction chunk
    int x_mt = b, x_kk = 0;
    // Round the finished tile into stage STG (consumed by every wave once the
    // step's middle barrier has passed; the next load into it is issued after
    // the closing barrier below), then store full pixel rows.  Rows are 128 B
    // with the 16-byte chunk XOR-ed by row & 7.
    auto epilogue = [&](auto stg) {
        constexpr int STG = decltype(stg)::value;
        unsigned char* tile = lds + STG * A_BYTES;
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j) {
                const int row = wm * (WMB * 16) + i * 16 + frow;
                const int col = wn * (WNB * 16) + j * 16 + fgrp * 4;
                const i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                                 int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
                *reinterpret_cast<i32x2*>(tile + row * kARow + (((col >> 3) ^ (row & 7)) << 4) +
                                          (col & 7) * 2) = v;
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int lim = min(a.bm, a.M - x_mt * a.bm);
        const int m0 = x_mt * a.bm;
#pragma unroll
        for (int q = 0; q < kPwBM * 8 / kThreads; ++q) {
            const int e = tid + q * kThreads;
            const int row = e >> 3, chunk = e & 7;
            const i32x4 v = *reinterpret_cast<const i32x4*>(tile + row * kARow + ((chunk ^ (row & 7)) << 4));
            if (row < lim && chunk * 8 < a.C)
                buf_store16(v, rdx, uint32_t(((m0 + row) * a.C + chunk * 8) * 2));
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // One reduction step out of stage STG, as in the ring kernel: first half
    // multiplies half 0 while reading half 1 and loading the step NS - 1
    // ahead into the stage freed by the previous step; wait for the next
    // stage; second half multiplies half 1 while reading the next step's
    // half 0.  After a tile's last step, its epilogue.
    constexpr int NM = WMB * WNB;
    constexpr int NI0 = NREAD + LOADS;
    constexpr int PER0 = (NI0 + NM - 1) / NM;
    constexpr int PER1 = (NREAD + NM - 1) / NM;
    auto step_fn = [&](auto stg) {
        constexpr int STG = decltype(stg)::value;
        constexpr int NXT = (STG + 1) % NS, FREE = (STG + NS - 1) % NS;
        const int nkk = x_kk + kBK >= a.kpad ? 0 : x_kk + kBK;
        const uint32_t w_cur = uint32_t(x_kk * B_ROW), w_nxt = uint32_t(nkk * B_ROW);
        sfor<NM>([&](auto mc) {
            constexpr int M = decltype(mc)::value;
            mfma_one(IC<0>{}, mc);
            sfor<PER0>([&](auto pc) {
                constexpr int X = M * PER0 + decltype(pc)::value;
                if constexpr (X < NREAD) read_one(stg, IC<1>{}, IC<X>{}, w_cur);
                else if constexpr (X < NI0) dma_one(IC<FREE>{}, IC<X - NREAD>{});
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        advance_i();
        wait_frags(IC<1>{});
        wait_vm<(NS - 2) * LOADS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        sfor<NM>([&](auto mc) {
            constexpr int M = decltype(mc)::value;
            mfma_one(IC<1>{}, mc);
            sfor<PER1>([&](auto pc) {
                constexpr int X = M * PER1 + decltype(pc)::value;
                if constexpr (X < NREAD) read_one(IC<NXT>{}, IC<0>{}, IC<X>{}, w_nxt);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        wait_frags(IC<0>{});
        if (nkk == 0) {
            epilogue(stg);
            x_mt += G;
        }
        x_kk = nkk;
    };

    if (steps > 0) {
        sfor<NS - 1>([&](auto sc) {
            sfor<LOADS>([&](auto dc) { dma_one(sc, dc); });
            advance_i();
        });
        wait_vm<(NS - 2) * LOADS>();   // the filter and stage 0
        __builtin_amdgcn_s_barrier();
        sfor<NREAD>([&](auto rc) { read_one(IC<0>{}, IC<0>{}, rc, 0u); });
        wait_frags(IC<0>{});
#pragma unroll 1
        for (int st = 0; st < steps; st += NS) {
            sfor<NS>([&](auto sc) {
                if (st + decltype(sc)::value < steps) step_fn(sc);
            });
        }
    }
    wait_vm<0>();   // loads issued past the last step still target LDS
}

// ---------------------------------------------------------------------------
// Pointwise (1x1) dgrad for C <= 64 and K in {64, 128, 192, 256}: per-wave
// row streaming.
//
// Same fragments and the same ascending 32-deep MFMA chain per output as the
// ring kernel (bit-identical results); the schedule is built around HBM
// access: every dY load instruction reads 1 KiB of contiguous memory (whole
// pixel rows), which streams markedly faster than the 128-byte row slices a
// 64-deep step of a wide tile touches.
//   * The filter (K x 64 channels) is loaded once per block and each wave
//     keeps all of it in registers as MFMA operand fragments.
//   * Each wave owns a contiguous run of M / waves pixels and walks it in
//     blocks of 16 pixels (16 whole dY rows, contiguous in memory) through a
//     private LDS ring: asynchronous loads write the rows straight into LDS,
//     several blocks ahead, with the 16-byte chunks of a row XOR-ed by
//     row & 7 (the permutation is applied to the source addresses, so the
//     loads stay contiguous) so the fragment reads are conflict-free.  No
//     other wave touches the ring: no barriers in the loop.
//   * A finished block is staged (rounded) in the slot it has just consumed
//     and written back as contiguous 16-byte runs of dX rows.
struct PwrArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int M, C, K;       // pixels, channels of dX (<= 64, multiple of 8), channels of dY (64*KC)
    int nwaves;        // waves in the grid
};

template <typename T, int KC, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void dgrad_pw_rows_kernel(const PwrArgs a) {
    constexpr int WNB = 4;                           // 64 channels: 4 MFMA column blocks
    constexpr int CPR = KC * 8;                      // 16-byte chunks per dY row
    constexpr int SLOT = 16 * CPR * 16;              // one 16-pixel block of dY rows
    constexpr int LPB = SLOT / 1024;                 // async loads per lane per block
    constexpr int W_BYTES = KC * kBK * kPwBN * 2;
    constexpr int NBF = (kPwLds - W_BYTES) / (WAVES * SLOT);
    constexpr int NB = NBF < 16 ? NBF : 16;          // ring slots per wave
    constexpr int RING = NB * SLOT;
    static_assert(NB >= 2, "ring depth");
    static_assert(W_BYTES + WAVES * RING <= kPwLds, "LDS");
    static_assert((NB - 1) * LPB < 64, "vmcnt range");
    static_assert(RING < 65536, "slot offsets fit the LDS immediate");
    static_assert(SLOT >= 16 * 128, "a slot holds the staged output block");
    __shared__ __attribute__((aligned(16))) unsigned char lds[W_BYTES + WAVES * RING];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frow = lane & 15, fgrp = lane >> 4;
    const int gw = blockIdx.x * WAVES + wave;
    const int r0 = int(int64_t(a.M) * gw / a.nwaves);
    const int r1 = int(int64_t(a.M) * (gw + 1) / a.nwaves);
    const int nblk = (r1 - r0 + 15) / 16;

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);
    unsigned char* ring = lds + W_BYTES + wave * RING;
    const uint32_t ring0 = lds_addr(ring);

    // ---- filter -> LDS: 1 KiB regions of 8 k-rows, chunks swizzled as in a
    // W stage; channels past C read as zeros ----
#pragma unroll
    for (int q = wave; q < KC * 8; q += WAVES) {
        const int row = 8 * q + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_b<8>(row);
        const uint32_t v = chunk * 8 < a.C ? uint32_t((row * a.C + chunk * 8) * 2) : kOob;
        dma16(rw, lds + q * 1024, v, 0);
    }

    // ---- dY block loads: load D of a block covers 1 KiB; lane l takes
    // element e = 64*D + l of the block (row e / CPR, stored chunk e % CPR,
    // holding source chunk (e % CPR) ^ (row & 7)) ----
    uint32_t a_voff[LPB];
    int a_row[LPB];
#pragma unroll
    for (int d = 0; d < LPB; ++d) {
        const int e = 64 * d + lane;
        const int r = e / CPR, p = e % CPR;
        a_row[d] = r;
        a_voff[d] = uint32_t((r * a.K + ((p ^ (r & 7)) * 8)) * 2);
    }
    auto issue = [&](auto slot, int blk) {
        constexpr int SL = decltype(slot)::value;
        (void)a_voff; (void)a_row;
        const int m0 = r0 + blk * 16;
        const int lim = r1 - m0;
        const uint32_t soff = uint32_t(m0) * uint32_t(a.K) * 2u;
#pragma unroll
        for (int d = 0; d < LPB; ++d)
            dma16(rdy, ring + SL * SLOT + d * 1024, a_row[d] < lim ? a_voff[d] : kOob, soff);
    };
    // every wave's filter loads go out before any dY block load, so the
    // filter (needed first, by all waves) is not queued behind dY blocks
    __builtin_amdgcn_s_barrier();
    sfor<NB - 1>([&](auto sc) { issue(sc, decltype(sc)::value); });

    // ---- filter fragments -> registers: lane (frow, fgrp) of fragment
    // (kc, ks, j) holds channel j*16 + frow, k-rows kc*64 + ks*32 + fgrp*8 .. +7 ----
    wait_vm<(NB - 1) * LPB>();
    __builtin_amdgcn_s_barrier();
    i32x4 wr[KC][2][WNB];
    {
        const uint32_t lds0 = lds_addr(lds);
        sfor<KC>([&](auto kcc) {
            constexpr int KCI = decltype(kcc)::value;
            (void)wr;
            i32x2 h[2][WNB][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < WNB; ++j)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int k = ks * 32 + fgrp * 8 + 4 * hh + (frow >> 2);
                        const int c = j * 16 + 4 * (frow & 3);
                        const uint32_t addr = lds0 + (KCI * kBK + k) * (kPwBN * 2) +
                                              (((c >> 3) ^ swz_b<8>(k)) << 4) + (c & 7) * 2;
                        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h[ks][j][hh]) : "v"(addr));
                    }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < WNB; ++j) {
                    asm volatile("" : "+v"(h[ks][j][0]), "+v"(h[ks][j][1]));
                    wr[KCI][ks][j] = i32x4{h[ks][j][0][0], h[ks][j][0][1], h[ks][j][1][0], h[ks][j][1][1]};
                }
        });
    }

    // fragment read addresses: lane (frow, fgrp) of half ks reads row frow,
    // chunk kc*8 + ks*4 + fgrp (stored at chunk ^ (frow & 7))
    uint32_t fa_addr[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        fa_addr[ks] = ring0 + frow * (CPR * 16) + (((ks * 4 + fgrp) ^ (frow & 7)) << 4);
    // output staging: lane (frow, fgrp) writes channels j*16 + fgrp*4 .. +3 of
    // pixel frow into 128-byte rows (16-byte chunks XOR-ed by row & 7) ...
    uint32_t st_addr[WNB];
#pragma unroll
    for (int j = 0; j < WNB; ++j)
        st_addr[j] = ring0 + frow * 128 + (((2 * j + (fgrp >> 1)) ^ (frow & 7)) << 4) + (fgrp & 1) * 8;
    // ... and reads back 16-byte chunk e = 64*d + lane of the block's
    // contiguous dX rows (row e / (C/8), chunk e % (C/8))
    const int cc = a.C / 8;
    uint32_t ld_addr[2];
    int ld_row[2], ld_e[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const int e = 64 * d + lane;
        const bool used = e < 16 * cc;
        const int r = used ? e / cc : 0, ch = used ? e % cc : 0;
        ld_e[d] = used ? e : -1;
        ld_row[d] = r;
        ld_addr[d] = ring0 + r * 128 + ((ch ^ (r & 7)) << 4);
    }

    auto block_fn = [&](auto slot, int blk) {
        constexpr int SL = decltype(slot)::value;
        (void)fa_addr; (void)st_addr; (void)ld_addr; (void)ld_row; (void)ld_e; (void)wr;
        issue(IC<(SL + NB - 1) % NB>{}, blk + NB - 1);
        wait_vm<(NB - 1) * LPB>();
        i32x4 af[KC][2];
        sfor<KC>([&](auto kcc) {
            constexpr int KCI = decltype(kcc)::value;
            (void)af; (void)fa_addr;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                asm volatile("ds_read_b128 %0, %1 offset:%2"
                             : "=v"(af[KCI][ks]) : "v"(fa_addr[ks]), "i"(SL * SLOT + KCI * 128));
        });
        f32x4 acc[WNB];
#pragma unroll
        for (int j = 0; j < WNB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        sfor<2 * KC>([&](auto xc) {
            constexpr int X = decltype(xc)::value, KCI = X / 2, KS = X % 2;
            (void)af; (void)acc; (void)wr;
            asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(af[KCI][KS]) : "i"(2 * KC - 1 - X));
#pragma unroll
            for (int j = 0; j < WNB; ++j)
                acc[j] = mfma16x16x32<T>(wr[KCI][KS][j], af[KCI][KS], acc[j]);
        });
        // round, stage in this slot, store contiguous dX rows
#pragma unroll
        for (int j = 0; j < WNB; ++j) {
            const i32x2 v = {int(pack2<T>(acc[j][0], acc[j][1])), int(pack2<T>(acc[j][2], acc[j][3]))};
            asm volatile("ds_write_b64 %0, %1 offset:%2" :: "v"(st_addr[j]), "v"(v), "i"(SL * SLOT));
        }
        const int m0 = r0 + blk * 16;
        const int lim = r1 - m0;
        i32x4 o[2];
#pragma unroll
        for (int d = 0; d < 2; ++d)
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(o[d]) : "v"(ld_addr[d]), "i"(SL * SLOT));
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(o[0]), "+v"(o[1]));
#pragma unroll
        for (int d = 0; d < 2; ++d)
            if (ld_e[d] >= 0 && ld_row[d] < lim)
                buf_store16(o[d], rdx, uint32_t((m0 * a.C + ld_e[d] * 8) * 2));
    };

#pragma unroll 1
    for (int b0 = 0; b0 < nblk; b0 += NB) {
        sfor<NB>([&](auto pc) {
            constexpr int P = decltype(pc)::value;
            if (b0 + P < nblk) block_fn(IC<P>{}, b0 + P);
        });
    }
    wait_vm<0>();   // loads issued past the last block still target LDS
}

// ---------------------------------------------------------------------------
// General dgrad with the dY operand staged as an LDS window (classes with at
// least two filter taps).
//
// A block owns a rectangle of th x tw pixels of one phase class of one image
// (and one 128- or 64-channel slice of dX).  Per 64-deep chunk of K, the dY
// window those pixels reach -- (th + nr - 1) x (tw + nt - 1) pixels -- is
// loaded into LDS once and every filter tap of the class reads a shifted view
// of it, so dY is fetched once per chunk instead of once per tap.  The window
// is stored as 8 planes, one per 16-byte group of 8 channels, each a dense
// array of window pixels: a tap shift is then a uniform offset of every lane's
// read address, and the 16 lanes of an MFMA row group read 16 consecutive
// 16-byte entries (no bank conflicts).  Two window buffers alternate between
// chunks; the window of chunk c+2 is requested once the last tap of chunk c
// has been read.
//
// The block runs 8 waves: two groups of 2 x 2 waves that compute the same
// output tile over alternate reduction steps (group g takes the steps with
// parity g).  One matrix-core wave per SIMD cannot issue MFMAs back to back;
// two waves per SIMD can, and each wave's LDS reads then overlap the other's
// matrix work.  W tiles stream through a 4-stage ring (each group loads its
// own steps); the groups' fp32 partial sums are added once at the end.  The
// reduction runs chunk-outer, tap-inner.
constexpr int kMaxQ = 7;          // 64-pixel groups per window plane (448 pixels)
constexpr int kHaloThreads = 512;
constexpr int kRing = 4;          // W ring stages of the window kernel
constexpr int kLdsMax = 160 * 1024;

struct HaloClass {
    int a, b;            // phase: h = a + s*hc, w = b + s*wc
    int hc, wc;          // class extents (rows, columns of dX in the class)
    int r0, t0, nr, nt;  // first filter row / column touching the class, and their counts
    int u_off, v_off;    // tap (0, 0) of class pixel (hc, wc) reads dY (hc + u_off, wc + v_off)
    int th, tw;          // tile rows / columns
    int bands_h, bands_w;
    int hw;              // window columns (tw + nt - 1)
    int hp;              // window plane entries (a multiple of 64)
    int tile_begin;      // first block of the class
    int nblocks;         // blocks of the class
    FastDiv fd_hw, fd_tw;  // division by hw and by tw
};

struct HaloArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, K, R, S, stride, Ho, Wo, Cg, Kg, G;
    int ctiles;
    int nclasses;
    int remap;
    uint32_t halo_bytes;  // one window buffer: 8 planes x hp x 16 bytes, maximum over classes
    HaloClass cls[kMaxClasses];
};

template <typename T, int WMB, int WNB, bool KR>
__global__ __launch_bounds__(kHaloThreads, 1) void dgrad_halo_kernel(const HaloArgs a) {
    constexpr int WAVES_N = 2;
    constexpr int BMC = 2 * WMB * 16;                   // tile capacity in pixels
    constexpr int BN = WAVES_N * WNB * 16;              // channels per tile
    constexpr int B_ROW = BN * 2;
    constexpr int B_CHUNKS = BN / 8;
    constexpr int B_BYTES = kBK * B_ROW;
    constexpr int B_REG = B_BYTES / 1024 / 4;           // loads per lane per stage (4 waves)
    constexpr int B_ROWS_PER_REG = 1024 / B_ROW;
    constexpr int C_STRIDE = BN * 2 + 16;
    static_assert(B_BYTES % 4096 == 0, "W stage splits over 4 waves");
    static_assert(3 * B_BYTES + 36 * B_ROW < 65536, "stage offsets fit the LDS immediate");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;   // reduction-step parity of this wave's group
    const int lw = wave & 3;     // wave within the group

    // ---- block -> (class, image, tile rectangle, group, channel slice) ----
    const int bid = blockIdx.x;
    int ci = 0;
#pragma unroll 1
    for (int i = 1; i < a.nclasses; ++i)
        if (bid >= a.cls[i].tile_begin) ci = i;
    const HaloClass cl = a.cls[ci];
    int local = bid - cl.tile_begin;
    if (a.remap) local = (local & 7) * (cl.nblocks >> 3) + (local >> 3);
    const int ct = local % a.ctiles;
    int rest = local / a.ctiles;
    const int g = rest % a.G;
    rest /= a.G;
    const int bw = rest % cl.bands_w;
    rest /= cl.bands_w;
    const int bh = rest % cl.bands_h;
    const int n = rest / cl.bands_h;
    const int hc0 = bh * cl.th, wc0 = bw * cl.tw;
    const int c0 = ct * BN;
    const int s = a.stride;
    const int nr = cl.nr, nt = cl.nt, hw = cl.hw, hp = cl.hp;

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // ---- per-lane window sources: lane covers window pixel i*64 + lane ----
    const int u_top = hc0 + cl.u_off - (nr - 1), v_left = wc0 + cl.v_off - (nt - 1);
    const int hreal = (cl.th + nr - 1) * hw;
    const int nq = hp >> 6;
    uint32_t hoff[kMaxQ];
#pragma unroll
    for (int i = 0; i < kMaxQ; ++i) {
        const int q = i * 64 + lane;
        hoff[i] = kOob;
        if (i < nq && q < hreal) {
            const int hy = fdiv(q, cl.fd_hw);
            const int u = u_top + hy, v = v_left + q - hy * hw;
            if (u >= 0 && u < a.Ho && v >= 0 && v < a.Wo)
                hoff[i] = uint32_t((((n * a.Ho + u) * a.Wo + v) * a.K + g * a.Kg) * 2);
        }
    }
    // window of chunk kc into buffer buf: wave w fills plane w
    auto issue_window = [&](int buf, int kc) {
        const int kk = kc * kBK;
        const int pl = wave;
        unsigned char* base = lds + buf * a.halo_bytes + pl * hp * 16;
        const uint32_t soff = uint32_t((kk + pl * 8) * 2);
        const bool kin = !KR || kk + pl * 8 < a.Kg;
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i)
            if (i < nq) dma16(rdy, base + i * 1024, kin ? hoff[i] : kOob, soff);
    };

    // ---- per-lane W sources: a group's 4 waves fill one stage ----
    const int wk_stride = a.R * a.S * a.Cg;
    uint32_t b_voff[B_REG];
#pragma unroll
    for (int i = 0; i < B_REG; ++i) {
        const int krow = B_ROWS_PER_REG * (lw + 4 * i) + lane / B_CHUNKS;
        const int chunk = (lane % B_CHUNKS) ^ swz_b<B_CHUNKS>(krow);
        b_voff[i] = c0 + chunk * 8 < a.Cg ? uint32_t((krow * wk_stride + chunk * 8) * 2) : kOob;
    }

    const int taps = nr * nt;
    const int kchunks = (a.Kg + kBK - 1) / kBK;
    const int steps = taps * kchunks;
    // With four or more taps, chunk 1 is first read after super-step 0, so its
    // window is requested then rather than delaying the first multiply.
    const bool defer1 = taps >= 4;
    // ring stage of step st is st % 4; this group's steps use stages grp and
    // grp + 2, so its ring base folds in grp and the rest is an immediate
    unsigned char* const ring_g = lds + 2 * a.halo_bytes + grp * B_BYTES;

    // W issue cursor of this group (uniform): tap (wi, wj), chunk offset wkk.
    // Past the last step it keeps producing in-range or range-checked loads
    // into stages that are never multiplied.
    int wi = 0, wj = 0, wkk = 0;
    auto advance_w = [&]() {
        ++wj;
        const bool w1 = wj >= nt;
        wj = w1 ? 0 : wj;
        wi += w1 ? 1 : 0;
        const bool w2 = wi >= nr;
        wi = w2 ? 0 : wi;
        wkk += w2 ? kBK : 0;
    };
    auto dma_w = [&](auto stg, auto ec) {
        constexpr int STG = decltype(stg)::value, E = decltype(ec)::value;
        (void)b_voff;
        const int rt = (cl.r0 + s * wi) * a.S + cl.t0 + s * wj;
        const uint32_t soff = uint32_t(((g * a.Kg + wkk) * wk_stride + rt * a.Cg + c0) * 2);
        uint32_t v = b_voff[E];
        if (KR) {
            const int krow = B_ROWS_PER_REG * (lw + 4 * E) + lane / B_CHUNKS;
            v = (wkk + krow < a.Kg) ? v : kOob;
        }
        dma16(rw, ring_g + STG * B_BYTES + (lw + 4 * E) * 1024, v, soff);
    };

    // ---- fragment read addresses ----
    const int wm = lw / WAVES_N, wn = lw % WAVES_N;
    const int frow = lane & 15, fgrp = lane >> 4;
    const uint32_t lds0 = lds_addr(lds);
    // Half 1 of a step reads planes 4..7 (a uniform offset of 4 planes) and
    // W k-rows 32..63; the second transpose read of a tile reads k-rows 4..7
    // further on.  The W swizzle depends only on k-row bits 0, 1 and 3, which
    // neither step changes, so both are immediate offsets.
    uint32_t fa_base[WMB];           // window buffer 0, half 0, tap (0, 0)
    uint32_t fb_addr[WNB];           // this group's first ring stage, half 0
#pragma unroll
    for (int i = 0; i < WMB; ++i) {
        const int m = wm * (WMB * 16) + i * 16 + frow;
        int q = (nr - 1) * hw + nt - 1;
        if (m < cl.th * cl.tw) {
            const int y = fdiv(m, cl.fd_tw);
            q += y * hw + m - y * cl.tw;
        }
        fa_base[i] = lds0 + uint32_t((fgrp * hp + q) * 16);
    }
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
        const int k = fgrp * 8 + (frow >> 2);
        const int c = wn * (WNB * 16) + j * 16 + 4 * (frow & 3);
        fb_addr[j] = lds_addr(ring_g) + k * B_ROW + (((c >> 3) ^ swz_b<B_CHUNKS>(k)) << 4) +
                     (c & 7) * 2;
    }
    const int plane4 = 4 * hp * 16;

    // read cursor of this group: tap (ri, rj) and chunk rkc of the own step
    // whose first half is read next; offset = window buffer - tap shift
    int ri = 0, rj = 0, rkc = 0;
    auto cursor_off = [&]() {
        return (rkc & 1) * int(a.halo_bytes) - (ri * hw + rj) * 16;
    };
    auto advance_r = [&]() {
        ++rj;
        const bool w1 = rj >= nt;
        rj = w1 ? 0 : rj;
        ri += w1 ? 1 : 0;
        const bool w2 = ri >= nr;
        ri = w2 ? 0 : ri;
        rkc += w2 ? 1 : 0;
    };

    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 fa[2][WMB];
    i32x2 fb[2][WNB][2];
    constexpr int NREAD = 2 * WNB + WMB;
    auto read_one = [&](auto stg, auto ksc, auto rc, int aoff) {
        constexpr int STG = decltype(stg)::value, KS = decltype(ksc)::value;
        constexpr int R = decltype(rc)::value;
        (void)fa; (void)fb; (void)fa_base; (void)fb_addr; (void)plane4;
        if constexpr (R < 2 * WNB) {
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(fb[KS][R / 2][R % 2])
                         : "v"(fb_addr[R / 2]),
                           "i"(STG * B_BYTES + KS * 32 * B_ROW + (R % 2) * 4 * B_ROW));
        } else {
            asm volatile("ds_read_b128 %0, %1"
                         : "=v"(fa[KS][R - 2 * WNB])
                         : "v"(fa_base[R - 2 * WNB] + uint32_t(aoff + KS * plane4)));
        }
    };
    auto wait_frags = [&](auto ksc) {
        constexpr int KS = decltype(ksc)::value;
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[KS][0]), "+v"(fb[KS][0][0]));
#pragma unroll
        for (int i = 1; i < WMB; ++i) asm volatile("" : "+v"(fa[KS][i]));
#pragma unroll
        for (int j = 0; j < WNB; ++j) asm volatile("" : "+v"(fb[KS][j][0]), "+v"(fb[KS][j][1]));
    };
    auto mfma_one = [&](auto ksc, auto mc) {
        constexpr int KS = decltype(ksc)::value, M = decltype(mc)::value;
        constexpr int i = M / WNB, j = M % WNB;
        const i32x4 b = {fb[KS][j][0][0], fb[KS][j][0][1], fb[KS][j][1][0], fb[KS][j][1][1]};
        acc[i][j] = mfma16x16x32<T>(b, fa[KS][i], acc[i][j]);
    };

    constexpr int NM = WMB * WNB;
    constexpr int PER0 = (NREAD + NM - 1) / NM;
    constexpr int NI1 = NREAD + B_REG;
    constexpr int PER1 = (NI1 + NM - 1) / NM;
    int off_cur = 0, off_next = 0;   // window offsets of this group's current and next step
    int end_step = taps - 1;         // last step of chunk end_chunk (block-uniform)
    int end_chunk = 0;
    // Super-step j: group g multiplies its step 2j + g.  First half: multiply
    // half 0 while reading half 1's fragments.  All waves then wait for their
    // own loads and meet at the barrier, after which every fragment of steps
    // <= 2j+1 has been read and every load issued before it has landed.
    // Second half: multiply half 1 while reading half 0 of the group's next
    // step and loading W of its step after that into the stage just freed.
    // A chunk whose last step was in this super-step frees its window buffer
    // for the chunk after next.
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
                    // loads first: they have until the next barrier but one to land
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
        wait_vm<B_REG>();   // the group's second stage may still be in flight
        __builtin_amdgcn_s_barrier();
        if (grp) advance_r();
        off_cur = cursor_off();
        advance_r();
        advance_r();
        off_next = cursor_off();
        sfor<NREAD>([&](auto rc) { read_one(IC<0>{}, IC<0>{}, rc, off_cur); });
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
    constexpr int NT = WMB * WNB;
    f32x4* part = reinterpret_cast<f32x4*>(lds) + lw * NT * 64 + lane;
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

    // ---- epilogue: round, stage the tile in LDS, 16-byte row stores ----
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j) {
                const int row = wm * (WMB * 16) + i * 16 + frow;
                const int col = wn * (WNB * 16) + j * 16 + fgrp * 4;
                i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                           int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
                *reinterpret_cast<i32x2*>(lds + row * C_STRIDE + col * 2) = v;
            }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;
    const int tpix = cl.th * cl.tw;
    for (int q = tid; q < BMC * CPR; q += kHaloThreads) {
        const int row = q / CPR, cc = q % CPR;
        const int c = c0 + cc * 8;
        if (row >= tpix || c >= a.Cg) continue;
        const int y = fdiv(row, cl.fd_tw);
        const int hc = hc0 + y, wc = wc0 + row - y * cl.tw;
        if (hc >= cl.hc || wc >= cl.wc) continue;
        const int pix = (n * a.H + cl.a + s * hc) * a.W + cl.b + s * wc;
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + row * C_STRIDE + cc * 16);
        buf_store16(v, rdx, uint32_t(pix * a.C + g * a.Cg + c) * 2u);
    }
}

// Tile shapes (M blocks per wave, N blocks per wave) on 2 x 2 waves:
//   0: 224-pixel capacity x 128 channels (deep channel counts)
//   1: 128 x 64 (narrow channel counts)
template <typename T, bool PW, bool KR, bool SK>
void launch_cfg(int cfg, const IgemmArgs& args, int blocks, hipStream_t st) {
    const dim3 grid(blocks, SK ? args.splits : 1);
    if (cfg == 0)
        hipLaunchKernelGGL((dgrad_igemm_kernel<T, 7, 4, PW, KR, SK>), grid, dim3(kThreads), 0, st, args);
    else
        hipLaunchKernelGGL((dgrad_igemm_kernel<T, 4, 2, PW, KR, SK>), grid, dim3(kThreads), 0, st, args);
}
template <typename T, bool PW>
void launch_kr(int cfg, bool kr, const IgemmArgs& args, int blocks, hipStream_t st) {
    if (args.splits > 1) {
        if (kr) launch_cfg<T, PW, true, true>(cfg, args, blocks, st);
        else launch_cfg<T, PW, false, true>(cfg, args, blocks, st);
        return;
    }
    if (kr) launch_cfg<T, PW, true, false>(cfg, args, blocks, st);
    else launch_cfg<T, PW, false, false>(cfg, args, blocks, st);
}

struct Cfg {
    int bmc, bn, per_cu;   // pixel capacity, channels, blocks resident per CU (LDS-bound)
};
constexpr Cfg kCfgs[2] = {{224, 128, 1}, {128, 64, 2}};

template <typename T, int NS, bool KR>
void launch_pw_inst(const PwArgs& a, size_t lds, hipStream_t st) {
    auto kern = dgrad_pw_persist_kernel<T, NS, KR>;
    static bool attr_set = false;   // the attribute is per kernel; idempotent if raced
    if (!attr_set) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPwLds);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(a.nblocks), dim3(kThreads), lds, st, a);
}
template <typename T, bool KR>
void launch_pw_ns(int ns, const PwArgs& a, size_t lds, hipStream_t st) {
    if (ns == 8) launch_pw_inst<T, 8, KR>(a, lds, st);
    else launch_pw_inst<T, 4, KR>(a, lds, st);
}

// dY ring depth of the persistent pointwise kernel: the deepest that fits
// beside the resident filter (0: the filter does not fit).
int pw_stages(int64_t k) {
    const int64_t wbytes = (k + kBK - 1) / kBK * kBK * kPwBN * 2;
    for (int ns : {8, 4})
        if (ns * int64_t(kPwStage) + wbytes <= kPwLds) return ns;
    return 0;
}

constexpr int kPwrWaves = 8;   // waves per block (two per SIMD)
template <typename T>
void launch_pwr_kc(int kc, const PwrArgs& a, int blocks, hipStream_t st) {
    constexpr int W = kPwrWaves;
    if (kc == 1) hipLaunchKernelGGL((dgrad_pw_rows_kernel<T, 1, W>), dim3(blocks), dim3(W * 64), 0, st, a);
    else if (kc == 2) hipLaunchKernelGGL((dgrad_pw_rows_kernel<T, 2, W>), dim3(blocks), dim3(W * 64), 0, st, a);
    else if (kc == 3) hipLaunchKernelGGL((dgrad_pw_rows_kernel<T, 3, W>), dim3(blocks), dim3(W * 64), 0, st, a);
    else hipLaunchKernelGGL((dgrad_pw_rows_kernel<T, 4, W>), dim3(blocks), dim3(W * 64), 0, st, a);
}

bool pw_rows_ok(const Prob& p) {
    return p.c <= kPwBN && p.c % 8 == 0 && p.k % kBK == 0 && p.k <= 4 * kBK;
}

// Row-streamed pointwise launch: one block per CU (at most), each wave over
// an equal run of pixels (at least 16 for small M).
int launch_pw_rows(const Prob& p, const void* dy, const void* w, void* dx, hipStream_t st) {
    PwrArgs a{};
    a.dy = dy; a.w = w; a.dx = dx;
    a.M = int(p.n * p.h * p.w);
    a.C = int(p.c); a.K = int(p.k);
    a.dy_bytes = uint32_t(int64_t(a.M) * a.K * 2);
    a.w_bytes = uint32_t(int64_t(a.K) * a.C * 2);
    a.dx_bytes = uint32_t(int64_t(a.M) * a.C * 2);
    if (a.M <= 0) return CNHWC_OK;
    const int blocks = int(std::min<int64_t>(kNumCUs, (a.M + 16 * kPwrWaves - 1) / (16 * kPwrWaves)));
    a.nwaves = blocks * kPwrWaves;
    const int kc = a.K / kBK;
    if (p.dtype == CNHWC_BF16) launch_pwr_kc<BF16>(kc, a, blocks, st);
    else launch_pwr_kc<F16>(kc, a, blocks, st);
    return CNHWC_OK;
}

// Persistent pointwise launch: one block per CU; tile height chosen so the
// tiles spread most evenly over the blocks.
int launch_pw_persist(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                      hipStream_t st) {
    PwArgs a{};
    a.dy = dy; a.w = w; a.dx = dx;
    a.M = int(p.n * p.h * p.w);
    a.C = int(p.c); a.K = int(p.k);
    a.kpad = (a.K + kBK - 1) / kBK * kBK;
    a.dy_bytes = uint32_t(int64_t(a.M) * a.K * 2);
    a.w_bytes = uint32_t(int64_t(a.K) * a.C * 2);
    a.dx_bytes = uint32_t(int64_t(a.M) * a.C * 2);
    const int64_t slots = kNumCUs;
    int best_bm = kPwBM;
    int64_t best_cost = INT64_MAX;
    for (int bm = kPwBM; bm >= kPwBM / 4; bm -= 2) {
        const int64_t tiles = (a.M + bm - 1) / bm;
        const int64_t cost = (tiles + slots - 1) / slots * bm;
        if (cost < best_cost) { best_cost = cost; best_bm = bm; }
    }
    // tune >= 16: tile height override (pixels per tile, at most the capacity)
    a.bm = pl.tune >= 16 ? std::min(pl.tune, kPwBM) : best_bm;
    const int64_t ntiles = (a.M + a.bm - 1) / a.bm;
    if (ntiles <= 0) return CNHWC_OK;
    a.ntiles = int(ntiles);
    a.nblocks = int(std::min<int64_t>(ntiles, slots));
    const int ns = pw_stages(a.K);
    const size_t lds = size_t(ns) * kPwStage + size_t(a.kpad) * kPwBN * 2;
    const bool bf = p.dtype == CNHWC_BF16;
    const bool kr = a.K % kBK != 0;
    if (bf) kr ? launch_pw_ns<BF16, true>(ns, a, lds, st) : launch_pw_ns<BF16, false>(ns, a, lds, st);
    else kr ? launch_pw_ns<F16, true>(ns, a, lds, st) : launch_pw_ns<F16, false>(ns, a, lds, st);
    return CNHWC_OK;
}

}  // namespace

std::string dgrad_igemm_reason(const Prob& p, bool pointwise) {
    if (pointwise) {
        if (p.r != 1 || p.s != 1) return "pointwise path needs a 1x1 filter";
        if (p.stride != 1) return "pointwise path needs stride 1";
        if (p.pad_h != 0 || p.pad_w != 0) return "pointwise path needs zero padding";
    }
    if (p.cg % 8 != 0) return "channels per group of dx must be a multiple of 8";
    if (p.kg % 8 != 0) return "channels per group of dy must be a multiple of 8";
    if (p.stride > 4) return "implicit-GEMM dgrad supports stride <= 4 (at most 16 phase classes)";
    {
        // the dY window of a one-pixel tile must fit the LDS window buffer
        const int64_t nr = (p.r + p.stride - 1) / p.stride, nt = (p.s + p.stride - 1) / p.stride;
        if (nr * nt > 384)
            return "implicit-GEMM dgrad needs ceil(R/stride)*ceil(S/stride) <= 384 (LDS window)";
    }
    if (p.ho * p.wo * p.k > (int64_t(1) << 30) || p.h * p.w * p.c > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    return "";
}

namespace {

template <typename T, int WMB, int WNB, bool KR>
void launch_halo_inst(const HaloArgs& a, int blocks, size_t lds, hipStream_t st) {
    auto kern = dgrad_halo_kernel<T, WMB, WNB, KR>;
    static bool attr_set = false;   // the attribute is per kernel; idempotent if raced
    if (!attr_set) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kHaloThreads), lds, st, a);
}

template <typename T>
void launch_halo_t(int cfg, bool kr, const HaloArgs& a, int blocks, size_t lds, hipStream_t st) {
    if (cfg == 0) {
        if (kr) launch_halo_inst<T, 7, 4, true>(a, blocks, lds, st);
        else launch_halo_inst<T, 7, 4, false>(a, blocks, lds, st);
    } else {
        if (kr) launch_halo_inst<T, 4, 2, true>(a, blocks, lds, st);
        else launch_halo_inst<T, 4, 2, false>(a, blocks, lds, st);
    }
}

// Window plane entries one buffer may hold: two buffers and the W ring share
// the LDS, and a lane covers at most kMaxQ window pixels.
int halo_hp_max(int bn) {
    return std::min(kMaxQ * 64, (kLdsMax - kRing * kBK * bn * 2) / (2 * 8 * 16) / 64 * 64);
}

// Tile rectangle of a class under a row cap: the widest column band (up to
// the whole class row) and then the most rows whose dY window fits a buffer.
bool halo_geometry(int hc, int wc, int nr, int nt, int bmc, int th_cap, int hp_max, int& th,
                   int& tw, int& hp) {
    nr = std::max(nr, 1);
    nt = std::max(nt, 1);
    for (tw = std::min(wc, bmc); tw >= 1; tw = tw > 8 ? tw - 8 : tw - 1) {
        for (th = std::min(std::min(hc, bmc / tw), th_cap); th >= 1; --th) {
            const int hreal = (th + nr - 1) * (tw + nt - 1);
            hp = (hreal + 63) / 64 * 64;
            if (hp <= hp_max) return true;
        }
    }
    return false;
}

// Launch the window kernel over the phase classes with at least two taps.
int launch_dgrad_halo(const Prob& p, const void* dy, const void* w, void* dx, hipStream_t st) {
    const int cfg = p.cg > 64 ? 0 : 1;
    const int BN = kCfgs[cfg].bn, BMC = kCfgs[cfg].bmc;
    const int hp_max = halo_hp_max(BN);
    HaloArgs a{};
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg); a.G = p.groups;
    a.ctiles = int((p.cg + BN - 1) / BN);
    const int s = p.stride;
    const int kchunks = int((p.kg + kBK - 1) / kBK);
    // phase classes, heaviest reduction first so long tiles start early
    HaloClass tmp[kMaxClasses];
    int nc = 0;
    for (int ca = 0; ca < s; ++ca)
        for (int cb = 0; cb < s; ++cb) {
            HaloClass c{};
            c.a = ca; c.b = cb;
            c.hc = int((p.h - ca + s - 1) / s);
            c.wc = int((p.w - cb + s - 1) / s);
            if (c.hc <= 0 || c.wc <= 0) continue;
            c.r0 = (ca + p.pad_h) % s;
            c.t0 = (cb + p.pad_w) % s;
            c.nr = c.r0 < p.r ? int((p.r - c.r0 + s - 1) / s) : 0;
            c.nt = c.t0 < p.s ? int((p.s - c.t0 + s - 1) / s) : 0;
            c.u_off = (ca + p.pad_h - c.r0) / s;
            c.v_off = (cb + p.pad_w - c.t0) / s;
            if (c.nr * c.nt >= 2) tmp[nc++] = c;
        }
    std::stable_sort(tmp, tmp + nc, [](const HaloClass& x, const HaloClass& y) {
        return x.nr * x.nt > y.nr * y.nt;
    });
    // Row cap: a block's time is set by its reduction (the tile capacity is
    // multiplied whatever its fill), so minimise the rounds of blocks over the
    // CUs, weighted by each class's steps; ties go to taller tiles.
    const int64_t slots = kNumCUs;
    int best_cap = BMC;
    int64_t best_cost = INT64_MAX;
    for (int cap = BMC; cap >= 1; --cap) {
        int64_t cost = 0;
        for (int i = 0; i < nc; ++i) {
            int th, tw, hp;
            if (!halo_geometry(tmp[i].hc, tmp[i].wc, tmp[i].nr, tmp[i].nt, BMC, cap, hp_max, th,
                               tw, hp))
                return CNHWC_UNSUPPORTED;
            const int64_t blocks = p.n * ((tmp[i].hc + th - 1) / th) * ((tmp[i].wc + tw - 1) / tw) *
                                   a.ctiles * a.G;
            cost += (blocks + slots - 1) / slots * std::max(1, tmp[i].nr * tmp[i].nt * kchunks);
        }
        if (cost < best_cost) { best_cost = cost; best_cap = cap; }
    }
    int total = 0;
    bool all8 = true;
    uint32_t halo_bytes = 0;
    for (int i = 0; i < nc; ++i) {
        HaloClass& c = tmp[i];
        halo_geometry(c.hc, c.wc, c.nr, c.nt, BMC, best_cap, hp_max, c.th, c.tw, c.hp);
        c.bands_h = (c.hc + c.th - 1) / c.th;
        c.bands_w = (c.wc + c.tw - 1) / c.tw;
        c.hw = c.tw + std::max(c.nt, 1) - 1;
        c.fd_hw = make_fastdiv(uint32_t(c.hw));
        c.fd_tw = make_fastdiv(uint32_t(c.tw));
        c.tile_begin = total;
        c.nblocks = int(p.n) * c.bands_h * c.bands_w * a.ctiles * a.G;
        if (c.nblocks % 8 != 0) all8 = false;
        total += c.nblocks;
        halo_bytes = std::max(halo_bytes, uint32_t(8 * c.hp * 16));
        a.cls[i] = c;
    }
    a.nclasses = nc;
    a.remap = all8 ? 1 : 0;
    a.halo_bytes = halo_bytes;
    if (total <= 0) return CNHWC_OK;
    const size_t ring = size_t(kRing) * kBK * BN * 2;
    const size_t epi = size_t(BMC) * (BN * 2 + 16);
    const size_t partials = size_t(BMC) * BN * 4;   // odd-step fp32 partial sums
    const size_t lds = std::max(std::max(2 * size_t(halo_bytes) + ring, epi), partials);
    const bool kr = p.kg % kBK != 0;
    if (p.dtype == CNHWC_BF16) launch_halo_t<BF16>(cfg, kr, a, total, lds, st);
    else launch_halo_t<F16>(cfg, kr, a, total, lds, st);
    return CNHWC_OK;
}

}  // namespace

// Split-K dgrad: reduction splits for a problem whose ring-kernel tiles
// cannot fill the GPU (1: do not split).  Deep reductions over few output
// tiles (small maps, many dY channels) split their steps so that tiles x
// splits blocks cover every compute unit once, each split at least 4 steps.
int dgrad_splitk_auto(const Prob& p) {
    const int cfg = p.cg > 64 ? 0 : 1;
    const int s = p.stride;
    int64_t tiles = 0, max_taps = 0;
    for (int ca = 0; ca < s; ++ca)
        for (int cb = 0; cb < s; ++cb) {
            const int64_t hc = (p.h - ca + s - 1) / s, wc = (p.w - cb + s - 1) / s;
            if (hc <= 0 || wc <= 0) continue;
            const int64_t r0 = (ca + p.pad_h) % s, t0 = (cb + p.pad_w) % s;
            const int64_t nr = r0 < p.r ? (p.r - r0 + s - 1) / s : 0;
            const int64_t nt = t0 < p.s ? (p.s - t0 + s - 1) / s : 0;
            tiles += (p.n * hc * wc + kCfgs[cfg].bmc - 1) / kCfgs[cfg].bmc *
                     ((p.cg + kCfgs[cfg].bn - 1) / kCfgs[cfg].bn) * p.groups;
            max_taps = std::max(max_taps, nr * nt);
        }
    const int64_t steps = max_taps * ((p.kg + kBK - 1) / kBK);
    if (tiles <= 0 || tiles >= kNumCUs / 2 || steps < 16) return 1;
    const int64_t sp = std::min<int64_t>({(kNumCUs + tiles - 1) / tiles, steps / 4, 64});
    if (sp > 1) {
        // a split is wanted: small maps take the filter-streaming kernel and its split count
        const int ss = dgrad_stream_splits(p);
        if (ss > 1 && dgrad_stream_reason(p, ss).empty()) return ss;
    }
    return int(std::max<int64_t>(sp, 1));
}

int launch_dgrad_igemm(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                       void* ws, hipStream_t st) {
    const bool sk = pl.variant == CNHWC_VAR_DGRAD_SPLITK;
    if (sk && (pl.split_c < 2 || ws == nullptr)) return CNHWC_UNSUPPORTED;
    // split-K over a small map: the filter-streaming kernel (any tune keeps
    // the ring kernel)
    if (dgrad_stream_taken(p, pl)) return launch_dgrad_stream(p, pl, dy, w, dx, ws, st);
    const bool pw = pl.variant == CNHWC_VAR_DGRAD_POINTWISE ||
                    (sk && p.r == 1 && p.s == 1 && p.stride == 1 && p.pad_h == 0 && p.pad_w == 0);
    // pointwise with C <= 64: the row-streamed kernel for K = 64..256 in
    // steps of 64, else the LDS-persistent kernel while the filter fits LDS
    // (tune 1 asks for the ring kernel, tune 3 or >= 16 for the LDS-persistent
    // one)
    if (pw && !sk && pl.tune != 1 && p.c <= kPwBN && p.groups == 1) {
        if (pw_rows_ok(p) && pl.tune != 3 && pl.tune < 16) return launch_pw_rows(p, dy, w, dx, st);
        if (pw_stages(p.k) > 0) return launch_pw_persist(p, pl, dy, w, dx, st);
    }
    // strided problems whose channel counts fit its tiles: the persistent
    // 8-wave kernel (tune 5 forces it, also at stride 1)
    if (!pw && !sk && dgrad_persist_taken(p, pl)) return launch_dgrad_persist(p, dy, w, dx, st);
    // Stride 1: classes with two or more taps go to the window kernel, the
    // rest (and the pointwise fast path) to the ring kernel below.  Strided
    // problems split into several classes of few taps each, where the window
    // kernel's fixed cost per block outweighs its dY reuse: ring kernel only.
    // (tune: 1 forces the ring kernel, 2 the window kernel.)
    const bool window = !pw && !sk && (pl.tune == 2 || (pl.tune != 1 && p.stride == 1));
    if (window) {
        const int rc = launch_dgrad_halo(p, dy, w, dx, st);
        if (rc != CNHWC_OK) return rc;
    }
    const int cfg = p.cg > 64 ? 0 : 1;
    const int BN = kCfgs[cfg].bn, BMC = kCfgs[cfg].bmc;
    IgemmArgs a{};
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.cg * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.K = int(p.k);
    a.R = int(p.r); a.S = int(p.s); a.stride = p.stride; a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.Ho = int(p.ho); a.Wo = int(p.wo); a.Cg = int(p.cg); a.Kg = int(p.kg); a.G = p.groups;
    a.ctiles = int((p.cg + BN - 1) / BN);
    a.splits = sk ? pl.split_c : 1;
    a.ws = sk ? static_cast<float*>(ws) : nullptr;
    const int s = p.stride;
    // phase classes, heaviest reduction first so long tiles start early
    struct C { ClassInfo ci; int64_t work; int64_t mc; };
    C tmp[kMaxClasses];
    int nc = 0;
    for (int ca = 0; ca < s; ++ca)
        for (int cb = 0; cb < s; ++cb) {
            ClassInfo ci{};
            ci.a = ca; ci.b = cb;
            ci.hc = int((p.h - ca + s - 1) / s);
            ci.wc = int((p.w - cb + s - 1) / s);
            if (ci.hc <= 0 || ci.wc <= 0) continue;
            ci.r0 = (ca + p.pad_h) % s;
            ci.t0 = (cb + p.pad_w) % s;
            ci.nr = ci.r0 < p.r ? int((p.r - ci.r0 + s - 1) / s) : 0;
            ci.nt = ci.t0 < p.s ? int((p.s - ci.t0 + s - 1) / s) : 0;
            ci.u_off = (ca + p.pad_h - ci.r0) / s;
            ci.v_off = (cb + p.pad_w - ci.t0) / s;
            ci.fd_hw = make_fastdiv(uint32_t(ci.hc * ci.wc));
            ci.fd_wc = make_fastdiv(uint32_t(ci.wc));
            if (!window || ci.nr * ci.nt <= 1)
                tmp[nc++] = C{ci, int64_t(ci.nr) * ci.nt, p.n * ci.hc * ci.wc};
        }
    std::stable_sort(tmp, tmp + nc, [](const C& x, const C& y) { return x.work > y.work; });
    // M tile.  A block's time grows with its capacity when the reduction is
    // long (matrix-core bound) and with its valid rows when it is short
    // (memory bound); pick the tile height that minimises rounds of blocks
    // over the block slots times that per-block cost.
    int64_t red = 0;
    for (int i = 0; i < nc; ++i) red = std::max(red, tmp[i].work * p.kg);
    const bool mem_bound = red <= 512;
    const int64_t slots = int64_t(kNumCUs) * kCfgs[cfg].per_cu;
    int best_bm = BMC;
    int64_t best_cost = INT64_MAX;
    for (int bm = BMC; bm >= std::max(16, BMC / 2); bm -= 2) {
        int64_t tiles = 0;
        for (int i = 0; i < nc; ++i) tiles += (tmp[i].mc + bm - 1) / bm * a.ctiles * a.G;
        const int64_t rounds = (tiles + slots - 1) / slots;
        const int64_t cost = rounds * (mem_bound ? bm : BMC);
        if (cost < best_cost) { best_cost = cost; best_bm = bm; }
    }
    a.bm = best_bm;
    // tune >= 16: tile height override (pixels per tile, at most the capacity)
    if (pl.tune >= 16) a.bm = std::min(pl.tune, BMC);
    int total = 0;
    bool all8 = true;
    for (int i = 0; i < nc; ++i) {
        tmp[i].ci.mtiles = int((tmp[i].mc + a.bm - 1) / a.bm);
        tmp[i].ci.tile_begin = total;
        const int cnt = tmp[i].ci.mtiles * a.ctiles * a.G;
        if (cnt % 8 != 0) all8 = false;
        total += cnt;
        a.cls[i] = tmp[i].ci;
    }
    a.nclasses = nc;
    a.remap = all8 ? 1 : 0;
    if (total <= 0) return CNHWC_OK;
    const bool bf = p.dtype == CNHWC_BF16;
    const bool kr = p.kg % kBK != 0;
    if (pw) bf ? launch_kr<BF16, true>(cfg, kr, a, total, st) : launch_kr<F16, true>(cfg, kr, a, total, st);
    else bf ? launch_kr<BF16, false>(cfg, kr, a, total, st) : launch_kr<F16, false>(cfg, kr, a, total, st);
    if (sk) {
        // second pass: dX = round(sum of the splits in ascending order), the
        // split-C forward's reduce over [split][N*H*W][C]
        Prob q = p;
        q.ho = p.h; q.wo = p.w; q.k = p.c;
        return launch_split_reduce(q, a.splits, ws, dx, st);
    }
    return CNHWC_OK;
}

}  // namespace cnhwc
