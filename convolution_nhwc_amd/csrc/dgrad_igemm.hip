// Backward-data convolution as implicit GEMMs on the gfx950 matrix cores,
// with the 1x1 pointwise fast path as a compile-time specialisation of the
// same tiling.
//
// Strided dgrad splits dX into stride*stride phase classes (h mod s, w mod s)
// -- the "tilde" decomposition of "perf(rocke/conv): add the pointwise fast
// path dgrad was missing" (Finding 4 and the fast-path commit).  In class
// (a, b) only the filter rows r = (a + pad_h) mod s + s*i and columns
// t = (b + pad_w) mod s + s*j touch dX, and dY row (h + pad_h - r)/s moves by
// exactly one row per step of i, so each class is a dense GEMM
//     dX_class[m, c] = sum_{i, j, k} dY[n, u0(m) - i, v0(m) - j, g*Kg + k] * W[g*Kg + k, r_i, t_j, c]
// with M = the class's pixels, N = Cg, and reduction Kg * taps.  Classes with
// no tap write zeros.  All classes run in one launch; a block finds its class
// in a small table in the kernel arguments (at most 16 scalar compares, no
// divide in the reduction loop).
//
// For 1x1, stride 1, no padding and one group the decomposition is the
// identity (one class, Hc = H, Wc = W, one tap) and the dY offset of GEMM row
// m is m*K + k and the W offset is k*C + c (same page, the fast-path commit).
// The PW specialisation uses exactly those offsets; everything else -- tiles,
// reduction order, MFMA sequence, rounding -- is shared, so it is bit-identical
// to the general kernel on the same problem.
//
// Tiling: 256 threads, BM x BN output tile, 64-deep reduction steps staged in
// LDS (double-buffered).  dY tiles load as 16-byte vectors along k; W tiles load
// as 16-byte vectors along c and are transposed in registers so that LDS holds
// both operands k-contiguous, as the MFMA operands need.  LDS rows are 128 bytes
// with the 16-byte chunks XOR-swizzled by (row & 7), so the fragment reads of
// eight consecutive rows hit distinct banks.  The MFMA computes the transposed
// tile (channels x pixels) so each lane ends with four consecutive channels of
// one pixel; the epilogue rounds to fp16/bf16 (RNE) and restages through LDS
// for full 16-byte row stores.  Out-of-range taps and rows read zero through
// the buffer descriptors' range check.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>

namespace cnhwc {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;        // reduction depth per LDS stage (halves)
constexpr int kRowBytes = 128; // kBK * 2
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
    int ctiles;        // ceil(Cg / BN)
    int nclasses;
    int remap;         // 1: remap block ids so each XCD works on contiguous tiles
    ClassInfo cls[kMaxClasses];
};

__device__ inline uint32_t swz(int row, int chunk) { return uint32_t((chunk ^ (row & 7)) * 16); }

template <typename T, int BM, int BN, bool PW>
__global__ __launch_bounds__(kThreads, 2) void dgrad_igemm_kernel(const IgemmArgs a) {
    constexpr int A_ROWS_PER_THREAD = BM * 8 / kThreads;      // 16-byte chunks of A per thread
    constexpr int KB_K = kBK * BN / (8 * kThreads);           // W rows per thread (x 8 channels)
    constexpr int WM = BM / 2, WN = BN / 2;                   // wave tile
    constexpr int FM = WM / 16, FN = WN / 16;                 // MFMA blocks per wave
    constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int C_STRIDE = BN * 2 + 16;
    static_assert(KB_K == 2 || KB_K == 4 || KB_K == 8, "tile");
    static_assert(BM * C_STRIDE <= 2 * STAGE, "epilogue tile must fit in LDS");
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // ---- block -> (class, m tile, group, c tile) ----
    int bid = blockIdx.x;
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

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // ---- per-thread A rows: dY base offset (elements) and tap origin ----
    const int a_chunk = tid & 7;
    int a_off[A_ROWS_PER_THREAD], a_u0[A_ROWS_PER_THREAD], a_v0[A_ROWS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < A_ROWS_PER_THREAD; ++i) {
        const int row = (tid >> 3) + i * (kThreads / 8);
        const int m = mt * BM + row;
        if (PW) {
            a_off[i] = m < Mc ? m * a.K : -1;
            a_u0[i] = 0;
            a_v0[i] = 0;
        } else if (m < Mc) {
            const int hw = cl.hc * cl.wc;
            const int n = m / hw;
            const int rem = m - n * hw;
            const int hc = rem / cl.wc;
            const int wc = rem - hc * cl.wc;
            const int u0 = (cl.a + s * hc + a.pad_h - cl.r0) / s;
            const int v0 = (cl.b + s * wc + a.pad_w - cl.t0) / s;
            a_u0[i] = u0;
            a_v0[i] = v0;
            a_off[i] = ((n * a.Ho + u0) * a.Wo + v0) * a.K + g * a.Kg;
        } else {
            a_off[i] = -1;
            a_u0[i] = -1 << 28;
            a_v0[i] = 0;
        }
    }
    // ---- per-thread W block: KB_K rows (k) x 8 channels ----
    const int b_cq = tid % (BN / 8);
    const int b_kq = tid / (BN / 8);
    const bool b_cvalid = c0 + b_cq * 8 < a.Cg;

    const int kchunks = (a.Kg + kBK - 1) / kBK;
    const int steps = cl.nr * cl.nt * kchunks;

    i32x4 ra[A_ROWS_PER_THREAD];
    i32x4 rb[KB_K];

    auto load_tile = [&](int step) {
        const int tap = step / kchunks;
        const int kk = (step - tap * kchunks) * kBK;
        const int ti = tap / cl.nt, tj = tap - ti * cl.nt;
        const int r = cl.r0 + s * ti, t = cl.t0 + s * tj;
        const bool kv = kk + a_chunk * 8 < a.Kg;
#pragma unroll
        for (int i = 0; i < A_ROWS_PER_THREAD; ++i) {
            uint32_t off = kOob;
            if (PW) {
                if (a_off[i] >= 0 && kv) off = uint32_t(a_off[i] + kk + a_chunk * 8) * 2u;
            } else {
                const int u = a_u0[i] - ti, v = a_v0[i] - tj;
                if (a_off[i] >= 0 && kv && u >= 0 && u < a.Ho && v >= 0 && v < a.Wo)
                    off = uint32_t(a_off[i] - (ti * a.Wo + tj) * a.K + kk + a_chunk * 8) * 2u;
            }
            ra[i] = buf_load16(rdy, off);
        }
#pragma unroll
        for (int j = 0; j < KB_K; ++j) {
            const int k = kk + b_kq * KB_K + j;
            uint32_t off = kOob;
            if (b_cvalid && k < a.Kg) {
                const int kglob = g * a.Kg + k;
                const int e = PW ? kglob * a.C + c0 + b_cq * 8
                                 : ((kglob * a.R + r) * a.S + t) * a.Cg + c0 + b_cq * 8;
                off = uint32_t(e) * 2u;
            }
            rb[j] = buf_load16(rw, off);
        }
    };

    auto store_tile = [&](int buf) {
        unsigned char* As = lds + buf * STAGE;
        unsigned char* Bs = As + A_BYTES;
#pragma unroll
        for (int i = 0; i < A_ROWS_PER_THREAD; ++i) {
            const int row = (tid >> 3) + i * (kThreads / 8);
            *reinterpret_cast<i32x4*>(As + row * kRowBytes + swz(row, a_chunk)) = ra[i];
        }
        // transpose the KB_K x 8 block (rows k, columns c) to 8 x KB_K
        const int kbase = b_kq * KB_K;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int crow = b_cq * 8 + c;
            uint32_t h[KB_K];
#pragma unroll
            for (int j = 0; j < KB_K; ++j) {
                const uint32_t word = uint32_t(rb[j][c >> 1]);
                h[j] = (c & 1) ? (word >> 16) : (word & 0xffffu);
            }
            unsigned char* dst = Bs + crow * kRowBytes + swz(crow, kbase >> 3) + (kbase & 7) * 2;
            if constexpr (KB_K == 2) {
                *reinterpret_cast<uint32_t*>(dst) = h[0] | (h[1] << 16);
            } else if constexpr (KB_K == 4) {
                i32x2 v = {int(h[0] | (h[1] << 16)), int(h[2] | (h[3] << 16))};
                *reinterpret_cast<i32x2*>(dst) = v;
            } else {
                i32x4 v = {int(h[0] | (h[1] << 16)), int(h[2] | (h[3] << 16)),
                           int(h[4] | (h[5] << 16)), int(h[6] | (h[7] << 16))};
                *reinterpret_cast<i32x4*>(dst) = v;
            }
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave >> 1, wn = wave & 1;
    const int frow = lane & 15, fgrp = lane >> 4;

    auto compute = [&](int buf) {
        const unsigned char* As = lds + buf * STAGE;
        const unsigned char* Bs = As + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int chunk = ks * 4 + fgrp;
            i32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WM + i * 16 + frow;
                fa[i] = *reinterpret_cast<const i32x4*>(As + row * kRowBytes + swz(row, chunk));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int crow = wn * WN + j * 16 + frow;
                fb[j] = *reinterpret_cast<const i32x4*>(Bs + crow * kRowBytes + swz(crow, chunk));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    // transposed product: rows = channels (W), columns = pixels (dY)
                    acc[i][j] = mfma16x16x32<T>(fb[j], fa[i], acc[i][j]);
        }
    };

    if (steps > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
#pragma unroll 1
        for (int st = 0; st < steps; ++st) {
            const bool more = st + 1 < steps;
            if (more) load_tile(st + 1);
            compute(st & 1);
            if (more) store_tile((st + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogue: round, stage the BM x BN tile in LDS, 16-byte row stores ----
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wm * WM + i * 16 + frow;            // pixel
            const int col = wn * WN + j * 16 + fgrp * 4;        // first of 4 channels
            i32x2 v = {int(pack2<T>(acc[i][j][0], acc[i][j][1])),
                       int(pack2<T>(acc[i][j][2], acc[i][j][3]))};
            *reinterpret_cast<i32x2*>(lds + row * C_STRIDE + col * 2) = v;
        }
    __syncthreads();
    constexpr int CPR = BN / 8;  // 16-byte chunks per row
#pragma unroll
    for (int q = tid; q < BM * CPR; q += kThreads) {
        const int row = q / CPR, cc = q % CPR;
        const int m = mt * BM + row;
        const int c = c0 + cc * 8;
        if (m >= Mc || c >= a.Cg) continue;
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

template <typename T, int BM, int BN, bool PW>
void launch_t(const IgemmArgs& args, int blocks, hipStream_t st) {
    hipLaunchKernelGGL((dgrad_igemm_kernel<T, BM, BN, PW>), dim3(blocks), dim3(kThreads), 0, st, args);
}

constexpr int kBM = 128;

int pick_bn(const Prob& p) { return p.cg > 64 ? 128 : 64; }

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
    const int BN = pick_bn(p);
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
    struct C { ClassInfo ci; int64_t work; };
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
            const int64_t mc = p.n * ci.hc * ci.wc;
            ci.mtiles = int((mc + kBM - 1) / kBM);
            tmp[nc++] = C{ci, int64_t(ci.nr) * ci.nt};
        }
    std::stable_sort(tmp, tmp + nc, [](const C& x, const C& y) { return x.work > y.work; });
    int total = 0;
    bool all8 = true;
    for (int i = 0; i < nc; ++i) {
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
    if (pw) {
        if (BN == 128) bf ? launch_t<BF16, kBM, 128, true>(a, total, st) : launch_t<F16, kBM, 128, true>(a, total, st);
        else bf ? launch_t<BF16, kBM, 64, true>(a, total, st) : launch_t<F16, kBM, 64, true>(a, total, st);
    } else {
        if (BN == 128) bf ? launch_t<BF16, kBM, 128, false>(a, total, st) : launch_t<F16, kBM, 128, false>(a, total, st);
        else bf ? launch_t<BF16, kBM, 64, false>(a, total, st) : launch_t<F16, kBM, 64, false>(a, total, st);
    }
    return CNHWC_OK;
}

}  // namespace cnhwc
