// Backward-data convolution as implicit GEMMs on the gfx950 matrix cores,
// with the 1x1 pointwise fast path as a compile-time specialisation of the
// same kernel.
//
// Strided dgrad splits dX into stride*stride phase classes (h mod s, w mod s)
// -- the "tilde" decomposition of "perf(rocke/conv): add the pointwise fast
// path dgrad was missing" (Finding 4 and the fast-path commit).  In class
// (a, b) only the filter rows r = (a + pad_h) mod s + s*i and columns
// t = (b + pad_w) mod s + s*j touch dX, and dY row (h + pad_h - r)/s moves by
// exactly one row per step of i, so each class is a dense GEMM
//     dX_class[m, c] = sum_{i, j, k} dY[n, u0(m) - i, v0(m) - j, g*Kg + k] * W[g*Kg + k, r_i, t_j, c]
// with M = the class's pixels, N = Cg, and reduction Kg * taps.  Classes with
// no tap write zeros.  All classes run in one launch, heaviest first; a block
// finds its class in a small table in the kernel arguments (a few scalar
// compares, no divide in the reduction loop).
//
// For 1x1, stride 1, no padding and one group the decomposition is the
// identity (one class, Hc = H, Wc = W, one tap): the dY offset of GEMM row m is
// m*K + k and the W offset is k*C + c (same page, the fast-path commit).  The PW
// specialisation uses exactly those offsets; the reduction order (ascending
// 32-deep MFMA steps with the same lane/k assignment) and the rounding are the
// same, so it is bit-identical to the general kernel on the same problem.
//
// Data path (gfx950): both operands go global -> LDS with asynchronous
// buffer loads that write LDS directly (no VGPR staging) into a ring of three
// stages, so two 64-deep reduction steps are in flight while one is
// multiplied.  dY tiles are 128-byte k-rows (16-byte chunks XOR-swizzled by
// row); W tiles keep their natural c-contiguous rows (chunks swizzled by k) and
// are read as MFMA operands with the LDS transpose read (ds_read_b64_tr_b16),
// which hands each lane four consecutive k of one channel.  Every per-lane
// address is computed once: in the loop, the uniform parts of the global
// offsets go in the scalar offset field and the stage offsets in the LDS
// instructions' immediate field (the loop is unrolled over the stages).  The
// MFMA computes the transposed tile (channels x pixels) so each lane ends with
// four consecutive channels of one pixel; the epilogue rounds to fp16/bf16
// (RNE) and restages through LDS for full 16-byte row stores.  Out-of-range
// taps, rows and channels read zero through the buffer descriptors' range check.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>
#include <type_traits>

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
    ClassInfo cls[kMaxClasses];
};

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Asynchronous 16-byte global -> LDS load: lane l writes lds_base + 16*l.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds_base, uint32_t voff,
                             uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) (lgkmcnt and expcnt left alone).
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

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

// LDS byte address (what ds_* instructions take) of a pointer into __shared__.
__device__ inline uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

template <int I>
using IC = std::integral_constant<int, I>;

template <typename T, int WMB, int WNB, bool PW>
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
#pragma unroll 1
    for (int i = 1; i < a.nclasses; ++i)
        if (bid >= a.cls[i].tile_begin) ci = i;
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
    // a_base: byte offset of the row's dY pixel at tap (0, 0) plus its chunk,
    // or -1 past the tile; a_umask / a_vmask: bit i (j) set when tap row i
    // (column j) of the class lands inside dY for this row.
    int a_base[A_REG];
    uint32_t a_umask[A_REG], a_vmask[A_REG];
    int a_kq[A_REG];
#pragma unroll
    for (int i = 0; i < A_REG; ++i) {
        const int row = 8 * (wave + 4 * i) + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_a(row);
        a_kq[i] = chunk * 8;
        const int m = m_lo + row;
        a_base[i] = -1;
        a_umask[i] = 0;
        a_vmask[i] = 0;
        if (row < a.bm && m < m_hi) {
            if (PW) {
                a_base[i] = (m * a.K + chunk * 8) * 2;
                a_umask[i] = a_vmask[i] = 1;
            } else {
                const int hw = cl.hc * cl.wc;
                const int n = m / hw;
                const int rem = m - n * hw;
                const int hc = rem / cl.wc;
                const int wc = rem - hc * cl.wc;
                const int u0 = (cl.a + s * hc + a.pad_h - cl.r0) / s;
                const int v0 = (cl.b + s * wc + a.pad_w - cl.t0) / s;
#pragma unroll 1
                for (int t = 0; t < cl.nr && t < 32; ++t)
                    if (u0 - t >= 0 && u0 - t < a.Ho) a_umask[i] |= 1u << t;
#pragma unroll 1
                for (int t = 0; t < cl.nt && t < 32; ++t)
                    if (v0 - t >= 0 && v0 - t < a.Wo) a_vmask[i] |= 1u << t;
                a_base[i] = (((n * a.Ho + u0) * a.Wo + v0) * a.K + g * a.Kg + chunk * 8) * 2;
            }
        }
    }
    // ---- per-lane B (W) sources: region q = wave + 4*i holds k-rows B_ROWS_PER_REG*q .. ----
    const int taps_rs = PW ? 1 : a.R * a.S;
    const int wk_stride = PW ? a.C : taps_rs * a.Cg;     // elements between W k-rows
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
    const bool k_ragged = (a.Kg % kBK) != 0;

    const int kchunks = (a.Kg + kBK - 1) / kBK;
    const int steps = cl.nr * cl.nt * kchunks;

    // A offsets of the current tap: recomputed (branch-free per lane) when a
    // step starts a new tap; the 64-element k offset goes in the scalar offset.
    uint32_t a_cur[A_REG];
    auto set_tap = [&](int ti, int tj) {
        const int tap_bytes = (ti * a.Wo + tj) * a.K * 2;
#pragma unroll
        for (int i = 0; i < A_REG; ++i) {
            const uint32_t bit = (a_umask[i] >> ti) & (a_vmask[i] >> tj) & 1u;
            a_cur[i] = bit ? uint32_t(a_base[i] - tap_bytes) : kOob;
        }
    };
    // issue the async loads of reduction step `step` into stage STG
    auto issue = [&](auto stg, int step) {
        constexpr int STG = decltype(stg)::value;
        const int tap = step / kchunks;
        const int kk = (step - tap * kchunks) * kBK;
        const int ti = PW ? 0 : tap / cl.nt;
        const int tj = PW ? 0 : tap - ti * cl.nt;
        if (!PW && kk == 0) set_tap(ti, tj);
        const uint32_t a_soff = uint32_t(kk * 2);
#pragma unroll
        for (int i = 0; i < A_REG; ++i) {
            uint32_t v = a_cur[i];
            if (k_ragged) v = (kk + a_kq[i] < a.Kg) ? v : kOob;
            dma16(rdy, lds + STG * A_BYTES + (wave + 4 * i) * 1024, v, a_soff);
        }
        int rt = 0;
        if (!PW) rt = (cl.r0 + s * ti) * a.S + cl.t0 + s * tj;
        const uint32_t b_soff = uint32_t(((g * a.Kg + kk) * wk_stride + rt * a.Cg + c0) * 2);
#pragma unroll
        for (int i = 0; i < B_REG; ++i) {
            uint32_t v = b_voff[i];
            if (k_ragged) v = (kk + b_krow[i] < a.Kg) ? v : kOob;
            dma16(rw, lds + B_BASE + STG * B_BYTES + (wave + 4 * i) * 1024, v, b_soff);
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

    i32x4 fa[2][WMB], fb[2][WNB];
    auto read_frags = [&](auto stg, auto ksc) {
        constexpr int STG = decltype(stg)::value, KS = decltype(ksc)::value;
#pragma unroll
        for (int j = 0; j < WNB; ++j) {
            i32x2 lo, hi;
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(lo) : "v"(fb_addr[KS][j][0]), "i"(STG * B_BYTES));
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(hi) : "v"(fb_addr[KS][j][1]), "i"(STG * B_BYTES));
            fb[KS][j] = i32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int i = 0; i < WMB; ++i) {
            i32x4 v;
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(v) : "v"(fa_addr[KS][i]), "i"(STG * A_BYTES));
            fa[KS][i] = v;
        }
    };
    // the LDS reads above are issued in asm, invisible to the compiler's wait
    // tracking: wait here and tie the fragments to the wait
    auto wait_frags = [&](auto ksc) {
        constexpr int KS = decltype(ksc)::value;
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(fa[KS][0]), "+v"(fb[KS][0]));
#pragma unroll
        for (int i = 1; i < WMB; ++i) asm volatile("" : "+v"(fa[KS][i]));
#pragma unroll
        for (int j = 1; j < WNB; ++j) asm volatile("" : "+v"(fb[KS][j]));
    };
    auto mfmas = [&](auto ksc) {
        constexpr int KS = decltype(ksc)::value;
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j)
                // transposed product: rows = channels (W), columns = pixels (dY)
                acc[i][j] = mfma16x16x32<T>(fb[KS][j], fa[KS][i], acc[i][j]);
    };

    // one reduction step out of stage STG
    auto step_fn = [&](auto stg, int st) {
        constexpr int STG = decltype(stg)::value;
        const int later = min(steps - 1 - st, kStages - 2);   // stages issued after st
        if (later >= 1) wait_vm<LOADS>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        read_frags(stg, IC<0>{});
        wait_frags(IC<0>{});
        read_frags(stg, IC<1>{});
        mfmas(IC<0>{});
        // the next loads go out while the matrix cores work through the batch
        if (st + kStages - 1 < steps) issue(IC<(STG + kStages - 1) % kStages>{}, st + kStages - 1);
        wait_frags(IC<1>{});
        mfmas(IC<1>{});
    };

    if (steps > 0) {
#pragma unroll
        for (int i = 0; i < A_REG; ++i) a_cur[i] = a_base[i] >= 0 ? uint32_t(a_base[i]) : kOob;
        issue(IC<0>{}, 0);
        if (steps > 1) issue(IC<1>{}, 1);
#pragma unroll 1
        for (int st = 0; st < steps; st += kStages) {
            step_fn(IC<0>{}, st);
            if (st + 1 < steps) step_fn(IC<1>{}, st + 1);
            if (st + 2 < steps) step_fn(IC<2>{}, st + 2);
        }
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
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
            const int n = m / hw;
            const int rem = m - n * hw;
            const int hc = rem / cl.wc;
            const int wc = rem - hc * cl.wc;
            pix = (n * a.H + cl.a + s * hc) * a.W + cl.b + s * wc;
        }
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + row * C_STRIDE + cc * 16);
        buf_store16(v, rdx, uint32_t(pix * a.C + g * a.Cg + c) * 2u);
    }
}

// Tile shapes (M blocks per wave, N blocks per wave) on 2 x 2 waves:
//   0: 224-pixel capacity x 128 channels (deep channel counts)
//   1: 128 x 64 (narrow channel counts)
template <typename T, bool PW>
void launch_cfg(int cfg, const IgemmArgs& args, int blocks, hipStream_t st) {
    if (cfg == 0)
        hipLaunchKernelGGL((dgrad_igemm_kernel<T, 7, 4, PW>), dim3(blocks), dim3(kThreads), 0, st, args);
    else
        hipLaunchKernelGGL((dgrad_igemm_kernel<T, 4, 2, PW>), dim3(blocks), dim3(kThreads), 0, st, args);
}

struct Cfg {
    int bmc, bn, per_cu;   // pixel capacity, channels, blocks resident per CU (LDS-bound)
};
constexpr Cfg kCfgs[2] = {{224, 128, 1}, {128, 64, 2}};

}  // namespace

std::string dgrad_igemm_reason(const Prob& p, bool pointwise) {
    if (pointwise) {
        if (p.r != 1 || p.s != 1) return "pointwise path needs a 1x1 filter";
        if (p.stride != 1) return "pointwise path needs stride 1";
        if (p.pad_h != 0 || p.pad_w != 0) return "pointwise path needs zero padding";
        if (p.groups != 1) return "pointwise path needs groups == 1";
    }
    if (p.cg % 8 != 0) return "channels per group of dx must be a multiple of 8";
    if (p.kg % 8 != 0) return "channels per group of dy must be a multiple of 8";
    if (p.stride > 4) return "implicit-GEMM dgrad supports stride <= 4 (at most 16 phase classes)";
    if (p.ho * p.wo * p.k > (int64_t(1) << 30) || p.h * p.w * p.c > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    return "";
}

int launch_dgrad_igemm(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                       hipStream_t st) {
    const bool pw = pl.variant == CNHWC_VAR_DGRAD_POINTWISE;
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
    if (pw) bf ? launch_cfg<BF16, true>(cfg, a, total, st) : launch_cfg<F16, true>(cfg, a, total, st);
    else bf ? launch_cfg<BF16, false>(cfg, a, total, st) : launch_cfg<F16, false>(cfg, a, total, st);
    return CNHWC_OK;
}

}  // namespace cnhwc
