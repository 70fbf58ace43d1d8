// Split-C direct forward for small output maps over deep channels, with the
// filter streamed once ("feat(rocke): split-C and grouped LDS-halo direct conv
// fwd kernels": the split_c variant -- the channel loop divided among
// workgroups, fp32 partial sums in a workspace, a second reduction pass; the
// layer it was made for, a small map with deep channels, has too few output
// tiles to fill the compute units).
//
// When the whole batch has few output pixels the filter dominates the
// traffic: at 7 x 7, 2048 -> 512 channels, 3 x 3, it is 18.9 MB against 1.6 MB
// of input and 0.4 MB of output.  A block here owns 32 output channels, one
// group of whole images (16 tiles of 16 pixels) and a contiguous range of
// input channels; the blocks that read the same filter lines run on one XCD,
// so each filter element is fetched from memory once.  The block walks its range
// in 32-channel chunks: a chunk's filter rows (32 output channels x R*S taps x
// 32 channels) and its input window for the group's images
// (((Ho-1)*s + R) x ((Wo-1)*s + S) pixels an image, zero outside the image)
// form one LDS stage, loaded with asynchronous loads that write LDS directly.
// Four stages hold two chunk pairs: the pair being multiplied and the next,
// whose loads are spread between the matrix instructions.
//
// The 8 waves split the work so that each LDS fragment feeds several matrix
// products: waves 0-3 multiply the even chunks of a pair and waves 4-7 the odd
// ones, and each wave computes both 16-channel row tiles against four
// 16-pixel tiles (8 MFMA 16x16x32 per tap from 2 filter and 4 window
// fragments).  Every tap reads a shifted view of the window.  At the end the
// odd-chunk waves hand their sums to the even-chunk waves through LDS, which
// add them in that fixed order and write the block's fp32 partial to
// ws[split][pixel][K]; the direct-forward file's reduce pass adds the splits
// in ascending order and rounds once.
//
// LDS rows are 64 bytes (32 channels); the four 16-byte chunks of row q are
// stored at chunk ^ ((q >> 2) & 3), so 16 consecutive rows read as one
// fragment fall on distinct banks.  The swizzle is applied through the load
// source addresses.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>

namespace cnhwc {
namespace {

constexpr int kSThreads = 512;
constexpr int kSKB = 32;          // output channels per block
constexpr int kSCK = 32;          // input channels per chunk
constexpr int kSRow = kSCK * 2;   // bytes per LDS row (one pixel or one filter row)
constexpr int kSSlots = 4;        // 16-pixel tiles per wave
constexpr int kSPartPx = 4 * kSSlots * 16;   // tile columns per image group (256)
constexpr int kSSlack = 2 * kSRow;            // LDS read past the last window (S - 1 <= 2 rows)
constexpr int kSStages = 4;
constexpr int kSLdsMax = 160 * 1024;
constexpr int kSMaxLoads = 8;     // 16-byte loads per lane per stage, filter and window each
constexpr int kSEpiBytes = 4 * 2 * kSSlots * 64 * 16;   // odd-chunk sums handed over
constexpr int kDgSpread = 5;      // dgrad form: taps over which a pair's loads are issued

struct StreamFwdArgs {
    const void* x;
    const void* w;
    float* ws;
    uint32_t x_bytes, w_bytes, ws_bytes;
    int H, W, C, K, stride, pad_h, pad_w, Ho, Wo;
    int M;              // N * Ho * Wo
    int IH, IW;         // window rows / columns per image
    int part_imgs;      // images per group
    int part_px;        // part_imgs * Ho * Wo
    int VW;             // tile grid row width: IW at stride 1, else Wo
    int part_vpx;       // part_imgs * Ho * VW tile-grid pixels
    int win_rows;       // part_imgs * IH * IW
    int wrow_bytes;     // filter region of a stage (R*S*32 rows)
    int stage_bytes;
    int x_loads;        // 16-byte window loads per lane per stage
    uint32_t wchunk_bytes;   // filter source advance per 32-channel chunk
    int ktiles, splits, csplit, npairs;
    int mparts, nblocks;   // image groups; ktiles * splits * mparts
    FastDiv fd_win, fd_iw, fd_hv, fd_vw;   // division by IH*IW, IW, Ho*VW, VW
};

__device__ inline int sw_chunk(int row) { return (row >> 2) & 3; }

// 64-bit LDS transpose read of 16-bit elements (ds_read_b64_tr_b16): within a
// 16-lane group, lane i gets element i % 4 ... of the four rows the group's
// lanes address, so 4 x 4 tiles come back transposed.
__device__ inline i32x2 lds_read_tr16(const unsigned char* p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(
        i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p));
}

// Workgroup barrier without the full wait for outstanding memory operations
// that __syncthreads() implies: the loads of the next chunk pair stay in
// flight across it (the waits the ring needs are explicit).  The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ inline void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// DG: the backward-data pass of a stride-1 convolution as this forward
// correlation (of dY, at padding R-1-pad, with the filter rotated by 180
// degrees and its two channel axes swapped).  The filter as stored has the
// output channels of that correlation contiguous, so a stage's filter rows
// are (tap, reduction channel) rows of 32 output channels, read back into the
// MFMA layout with the LDS transpose read.
template <typename T, int TAPS, bool DG>
__global__ __launch_bounds__(kSThreads, 1) void fwd_stream_kernel(const StreamFwdArgs a) {
    constexpr int kS = TAPS == 9 ? 3 : 1;           // filter width
    constexpr int kWRows = TAPS * kSKB;             // filter rows of a stage
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2;    // chunk parity this wave multiplies
    const int grp = wave & 3;      // its tiles: 4 grp .. 4 grp + 3 of the image group

    // block -> (image group, k tile, split).  Blocks are dealt to the 8 XCDs
    // round-robin; the remap gives each XCD a contiguous run of the order
    // (split, k tile, image group), so the image groups of a k tile and
    // neighbouring k tiles -- the blocks that read the same filter lines (the
    // same 128-byte lines of a dgrad filter row hold two k tiles) -- and one
    // split's input channels share an L2
    int lb = blockIdx.x;
    if ((a.nblocks & 7) == 0) lb = (lb & 7) * (a.nblocks >> 3) + (lb >> 3);
    const int mp = lb % a.mparts;
    const int rest = lb / a.mparts;
    const int kt = rest % a.ktiles;
    const int sp = rest / a.ktiles;
    const int k0 = kt * kSKB;
    const int c_lo = sp * a.csplit;
    const int img0 = mp * a.part_imgs;

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rws = make_rsrc(a.ws, a.ws_bytes);

    // ---- load sources: slot e of a stage region is its row e / 4, 16-byte
    // position e % 4 (holding source chunk position ^ swizzle); the chunk's
    // channel offset goes in the scalar offset ----
    constexpr int wslots = kWRows * 4;
    constexpr int kWLoads = (wslots + kSThreads - 1) / kSThreads;
    const int xslots = a.win_rows * 4;
    const int per_img = a.IH * a.IW;
    uint32_t wsrc[kSMaxLoads], xsrc[kSMaxLoads];
#pragma unroll
    for (int i = 0; i < kSMaxLoads; ++i) {
        const int e = i * kSThreads + tid;
        wsrc[i] = kOob;
        if (i < kWLoads && e < wslots) {
            const int row = e >> 2, pos = e & 3;
            const int tap = row / kSKB, k = row - tap * kSKB;
            if constexpr (DG)   // row (tap, reduction channel c_lo + k): 32 output channels from k0
                wsrc[i] = uint32_t(((size_t(c_lo + k) * TAPS + (TAPS - 1 - tap)) * a.K + k0 +
                                    (pos ^ sw_chunk(row)) * 8) * 2);
            else                // row (tap, output channel k0 + k): 32 reduction channels from c_lo
                wsrc[i] = uint32_t(((size_t(k0 + k) * TAPS + tap) * a.C + c_lo + (pos ^ sw_chunk(row)) * 8) * 2);
        }
        xsrc[i] = kOob;
        if (i < a.x_loads && e < xslots) {
            const int row = e >> 2, pos = e & 3;
            const int img = fdiv(row, a.fd_win);
            const int rem = row - img * per_img;
            const int iy = fdiv(rem, a.fd_iw), ix = rem - iy * a.IW;
            const int h = iy - a.pad_h, w = ix - a.pad_w;
            if (h >= 0 && h < a.H && w >= 0 && w < a.W)
                xsrc[i] = uint32_t(((size_t((img0 + img) * a.H + h) * a.W + w) * a.C + c_lo +
                                    (pos ^ sw_chunk(row)) * 8) * 2);
        }
    }

    // The loads of a chunk pair, as one list of kQ instructions a lane: the
    // filter loads of its two stages, then their window loads.  Load q of
    // pair jj goes out while pair jj-1 is multiplied, after the products of
    // tap q % TAPS: spread between the matrix instructions, they never hold
    // up a wave.  (The dgrad form issues them over the first taps instead:
    // measured 23.0 against 25.2 us on its split-K workload; the forward is
    // fastest with the even spread.)  A lane past a region's end loads nothing (its LDS slot
    // would be the next region's).
    constexpr int kQ = 2 * (kWLoads + kSMaxLoads);
    auto issue_one = [&](auto qc, int jj) {
        constexpr int q = decltype(qc)::value;
        if (jj >= a.npairs) return;
        const int set = (jj & 1) * 2;
        if constexpr (q < 2 * kWLoads) {
            constexpr int h = q / kWLoads, i = q % kWLoads;
            if (i * kSThreads + tid < wslots)
                dma16(rw, lds + (set + h) * a.stage_bytes + (i * kSThreads + wave * 64) * 16, wsrc[i],
                      uint32_t(2 * jj + h) * a.wchunk_bytes);
        } else {
            constexpr int h = (q - 2 * kWLoads) / kSMaxLoads, i = (q - 2 * kWLoads) % kSMaxLoads;
            if (i < a.x_loads && i * kSThreads + tid < xslots)
                dma16(rx, lds + (set + h) * a.stage_bytes + a.wrow_bytes + (i * kSThreads + wave * 64) * 16,
                      xsrc[i], uint32_t((2 * jj + h) * kSCK * 2));
        }
    };
    // pair 0: in flight while the fragment addresses are worked out
    sfor<kQ>([&](auto qc) { issue_one(qc, 0); });

    // ---- fragment addresses.  The pixel tiles run over a grid of Ho rows of
    // VW columns an image: at stride 1 VW is the window width, so a tile's 16
    // pixels sit on 16 consecutive window rows for every tap (conflict-free
    // LDS reads) and the S - 1 extra columns a row are computed and dropped.
    // Window: tile slot i is grid tile 4 grp + i; the lane reads grid pixel
    // 16 * tile + lane % 16 at window row q(pixel) + tap shift, chunk
    // lane / 16.  Filter: row tap * 32 + 16 f + lane % 16 ----
    const int g = lane >> 4, r16 = lane & 15;
    const int s = a.stride;
    uint32_t xaddr[kSSlots][TAPS];
#pragma unroll
    for (int i = 0; i < kSSlots; ++i) {
        int m = (grp * kSSlots + i) * 16 + r16;
        if (m >= a.part_vpx) m = 0;                  // a valid row; the sums are never stored
        const int img = fdiv(m, a.fd_hv);
        const int rem = m - img * (a.Ho * a.VW);
        const int oy = fdiv(rem, a.fd_vw), ox = rem - oy * a.VW;
        const int q0 = img * per_img + oy * s * a.IW + ox * s;
#pragma unroll
        for (int t = 0; t < TAPS; ++t) {
            const int q = q0 + (t / kS) * a.IW + (t % kS);
            xaddr[i][t] = uint32_t(a.wrow_bytes + q * kSRow + ((g ^ sw_chunk(q)) << 4));
        }
    }
    // rows t * 32 + 16 f + r16 all swizzle by (r16 >> 2) & 3
    const uint32_t wlane = uint32_t(r16 * kSRow + ((g ^ sw_chunk(r16)) << 4));
    // DG: fragment (t, f) of lane (r16, g) is output channel 16 f + r16,
    // reduction channels 8 g .. 8 g + 7: two transposed reads of 4 rows
    // (t * 32 + 8 g + 4 hh + r16 / 4) x 4 channels (16 f + 4 (r16 % 4)); those
    // rows swizzle by (2 g + hh) & 3
    uint32_t wtr[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int q = r16 & 3;
            wtr[f][hh] = uint32_t((8 * g + 4 * hh + (r16 >> 2)) * kSRow +
                                  (((2 * f + (q >> 1)) ^ ((2 * g + hh) & 3)) << 4) + (q & 1) * 8);
        }
    auto read_w = [&](const unsigned char* sb, int t, int f) -> i32x4 {
        if constexpr (DG) {
            const i32x2 lo = lds_read_tr16(sb + t * kSKB * kSRow + wtr[f][0]);
            const i32x2 hi = lds_read_tr16(sb + t * kSKB * kSRow + wtr[f][1]);
            return i32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            return *reinterpret_cast<const i32x4*>(sb + wlane + (t * 2 + f) * 16 * kSRow);
        }
    };

    f32x4 acc[2][kSSlots];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int i = 0; i < kSSlots; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
    for (int j = 0; j < a.npairs; ++j) {
        // this wave's loads of pair j (the only ones in flight) have landed;
        // after the barrier everyone's have, and everyone is done with pair
        // j-1, whose stages pair j+1 fills from here on
        wait_vm<0>();
        ring_barrier();
        const unsigned char* sb = lds + ((j & 1) * 2 + half) * a.stage_bytes;
        // tap by tap; the next tap's fragments are read before this tap's
        // products, which update 8 different accumulators
        i32x4 wf[2][2], xf[2][kSSlots];
#pragma unroll
        for (int f = 0; f < 2; ++f) wf[0][f] = read_w(sb, 0, f);
#pragma unroll
        for (int i = 0; i < kSSlots; ++i) xf[0][i] = *reinterpret_cast<const i32x4*>(sb + xaddr[i][0]);
        sfor<TAPS>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int cur = t & 1, nxt = cur ^ 1;
            if constexpr (t + 1 < TAPS) {
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    wf[nxt][f] = read_w(sb, t + 1, f);
#pragma unroll
                for (int i = 0; i < kSSlots; ++i)
                    xf[nxt][i] = *reinterpret_cast<const i32x4*>(sb + xaddr[i][t + 1]);
            }
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int i = 0; i < kSSlots; ++i)   // rows = output channels, columns = pixels
                    acc[f][i] = mfma16x16x32<T>(wf[cur][f], xf[cur][i], acc[f][i]);
            if constexpr (DG) {
                // the dgrad filter chunks each open their own 128-byte line:
                // the next pair's loads go out over the first kDgSpread taps
                constexpr int NSP = TAPS < kDgSpread ? TAPS : kDgSpread;
                if constexpr (t < NSP) {
                    constexpr int q0 = t * kQ / NSP, q1 = (t + 1) * kQ / NSP;
                    sfor<q1 - q0>([&](auto uc) { issue_one(IC<q0 + decltype(uc)::value>{}, j + 1); });
                }
            } else {
                sfor<(kQ - t + TAPS - 1) / TAPS>([&](auto uc) { issue_one(IC<t + TAPS * decltype(uc)::value>{}, j + 1); });
            }
        });
    }

    // ---- odd-chunk sums to the even-chunk waves, then the block's fp32
    // partial: lane holds channels k0 + 16 f + 4 g .. +3 of pixel
    // 16 * tile + lane % 16 ----
    __syncthreads();   // every stage is read
    f32x4* hand = reinterpret_cast<f32x4*>(lds);
    if (half == 1) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int i = 0; i < kSSlots; ++i) hand[((grp * 2 + f) * kSSlots + i) * 64 + lane] = acc[f][i];
    }
    __syncthreads();
    if (half == 0) {
        const int64_t row0 = int64_t(sp) * a.M + int64_t(mp) * a.part_px;
#pragma unroll
        for (int i = 0; i < kSSlots; ++i) {
            const int m = (grp * kSSlots + i) * 16 + r16;
            const int img = fdiv(m, a.fd_hv);
            const int rem = m - img * (a.Ho * a.VW);
            const int oy = fdiv(rem, a.fd_vw), ox = rem - oy * a.VW;
            const bool in = m < a.part_vpx && ox < a.Wo;
            const int64_t row = row0 + (img * a.Ho + oy) * a.Wo + ox;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const f32x4 v = acc[f][i] + hand[((grp * 2 + f) * kSSlots + i) * 64 + lane];
                const int k = k0 + 16 * f + 4 * g;
                buf_store16(__builtin_bit_cast(i32x4, v), rws, in ? uint32_t((row * a.K + k) * 4) : kOob);
            }
        }
    }
}

// LDS bytes of one stage with groups of `imgs` images, 0 if such a group
// does not fit the block (pixels, per-lane load counts, four stages in LDS).
int64_t stream_stage_bytes(const Prob& p, int64_t imgs) {
    const int64_t IH = (p.ho - 1) * p.stride + p.r, IW = (p.wo - 1) * p.stride + p.s;
    if (imgs * p.ho * (p.stride == 1 ? IW : p.wo) > kSPartPx) return 0;
    const int64_t win_rows = imgs * IH * IW;
    const int64_t w_loads = (p.r * p.s * kSKB * 4 + kSThreads - 1) / kSThreads;
    const int64_t x_loads = (win_rows * 4 + kSThreads - 1) / kSThreads;
    if (w_loads > kSMaxLoads || x_loads > kSMaxLoads) return 0;
    const int64_t stage = (p.r * p.s * kSKB + win_rows) * kSRow;
    if (std::max<int64_t>(kSStages * stage + kSSlack, kSEpiBytes) > kSLdsMax) return 0;
    return stage;
}

// Image groups: the fewest that fit the block (0 if none).
int stream_parts(const Prob& p) {
    for (int64_t d = 1; d <= p.n; ++d)
        if (p.n % d == 0 && stream_stage_bytes(p, p.n / d) > 0) return int(d);
    return 0;
}

bool stream_geometry(const Prob& p, int splits, StreamFwdArgs* a, size_t* lds) {
    if (p.groups != 1) return false;
    const int taps = int(p.r * p.s);
    if (!((p.r == 1 && p.s == 1) || (p.r == 3 && p.s == 3))) return false;
    if (p.k % kSKB != 0) return false;
    const int mparts = stream_parts(p);
    if (mparts == 0) return false;
    if (splits < 1 || p.c % splits != 0 || (p.c / splits) % (2 * kSCK) != 0) return false;
    const int64_t part_imgs = p.n / mparts;
    const int64_t IH = (p.ho - 1) * p.stride + p.r, IW = (p.wo - 1) * p.stride + p.s;
    const int64_t win_rows = part_imgs * IH * IW;
    const int64_t x_loads = (win_rows * 4 + kSThreads - 1) / kSThreads;
    const int64_t stage = stream_stage_bytes(p, part_imgs);
    const int64_t need = std::max<int64_t>(kSStages * stage + kSSlack, kSEpiBytes);
    const int64_t M = p.n * p.ho * p.wo;
    if (int64_t(splits) * M * p.k * 4 > kBufferLimit) return false;
    a->H = int(p.h); a->W = int(p.w); a->C = int(p.c); a->K = int(p.k);
    a->stride = p.stride; a->pad_h = p.pad_h; a->pad_w = p.pad_w;
    a->Ho = int(p.ho); a->Wo = int(p.wo); a->M = int(M);
    a->IH = int(IH); a->IW = int(IW);
    a->part_imgs = int(part_imgs);
    a->part_px = int(part_imgs * p.ho * p.wo);
    a->VW = int(p.stride == 1 ? IW : p.wo);
    a->part_vpx = int(part_imgs * p.ho * a->VW);
    a->win_rows = int(win_rows);
    a->wrow_bytes = taps * kSKB * kSRow;
    a->stage_bytes = int(stage);
    a->x_loads = int(x_loads);
    a->ktiles = int(p.k / kSKB);
    a->splits = splits;
    a->csplit = int(p.c / splits);
    a->npairs = a->csplit / (2 * kSCK);
    a->mparts = mparts;
    a->nblocks = a->ktiles * splits * mparts;
    a->fd_win = make_fastdiv(uint32_t(IH * IW));
    a->fd_iw = make_fastdiv(uint32_t(IW));
    a->fd_hv = make_fastdiv(uint32_t(p.ho * a->VW));
    a->fd_vw = make_fastdiv(uint32_t(a->VW));
    *lds = size_t(need);
    return true;
}

template <typename T, bool DG>
int launch_taps(int taps, const StreamFwdArgs& a, size_t lds, int blocks, hipStream_t st) {
    auto set_lds = [&](const void* fn) {
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kSLdsMax) == hipSuccess;
    };
    switch (taps) {
    case 1: {
        static bool ok = set_lds(reinterpret_cast<const void*>(&fwd_stream_kernel<T, 1, DG>));
        if (!ok) return CNHWC_HIP_ERROR;
        hipLaunchKernelGGL((fwd_stream_kernel<T, 1, DG>), dim3(blocks), dim3(kSThreads), lds, st, a);
        return CNHWC_OK;
    }
    case 9: {
        static bool ok = set_lds(reinterpret_cast<const void*>(&fwd_stream_kernel<T, 9, DG>));
        if (!ok) return CNHWC_HIP_ERROR;
        hipLaunchKernelGGL((fwd_stream_kernel<T, 9, DG>), dim3(blocks), dim3(kSThreads), lds, st, a);
        return CNHWC_OK;
    }
    default: return CNHWC_UNSUPPORTED;
    }
}

}  // namespace

// Splits for the streaming kernel: one block per compute unit.
int fwd_stream_splits(const Prob& p) {
    if (p.k % kSKB != 0) return 0;
    const int mparts = stream_parts(p);
    if (mparts == 0) return 0;
    const int64_t blocks1 = (p.k / kSKB) * mparts;
    if (blocks1 > kNumCUs / 2) return 0;
    int sp = int(kNumCUs / blocks1);
    while (sp > 1 && (p.c % sp != 0 || (p.c / sp) % (2 * kSCK) != 0)) --sp;
    return sp >= 2 ? sp : 0;
}

std::string fwd_stream_reason(const Prob& p, int splits) {
    if (p.groups != 1) return "the filter-streaming split-C kernel needs groups == 1";
    if (!((p.r == 1 && p.s == 1) || (p.r == 3 && p.s == 3)))
        return "the filter-streaming split-C kernel has 1x1 and 3x3 instances";
    if (stream_parts(p) == 0)
        return "the filter-streaming split-C kernel needs the images split into groups of at most 256 "
               "tile pixels whose input windows fit LDS";
    StreamFwdArgs a{};
    size_t lds;
    if (!stream_geometry(p, splits, &a, &lds))
        return "the filter-streaming split-C kernel needs K a multiple of 32 and C/splits a multiple of 64";
    return "";
}

int launch_fwd_stream(const Prob& p, const Plan& pl, const void* x, const void* w, void* y, void* ws,
                      hipStream_t st) {
    StreamFwdArgs a{};
    size_t lds;
    if (!stream_geometry(p, pl.split_c, &a, &lds)) return CNHWC_UNSUPPORTED;
    a.x = x; a.w = w; a.ws = static_cast<float*>(ws);
    a.x_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.c * 2);
    a.ws_bytes = uint32_t(int64_t(a.splits) * a.M * p.k * 4);
    a.wchunk_bytes = uint32_t(kSCK * 2);
    const int blocks = a.nblocks;
    const int rc = p.dtype == CNHWC_BF16 ? launch_taps<BF16, false>(int(p.r * p.s), a, lds, blocks, st)
                                         : launch_taps<F16, false>(int(p.r * p.s), a, lds, blocks, st);
    if (rc != CNHWC_OK) return rc;
    return launch_split_reduce(p, a.splits, ws, y, st);
}

// ---- backward data through the same kernel ([PW] split-K: the dgrad of a
// layer with few output pixels over a deep reduction) ----

namespace {
// The stride-1 dgrad as a forward problem: input dY (Ho x Wo x K), output dX
// (H x W x C), padding R-1-pad, filter rotated with its channel axes swapped.
Prob dgrad_stream_view(const Prob& p) {
    Prob q = p;
    q.h = p.ho; q.w = p.wo; q.ho = p.h; q.wo = p.w;
    q.c = p.k; q.k = p.c; q.cg = p.k; q.kg = p.c;
    q.pad_h = int(p.r) - 1 - p.pad_h;
    q.pad_w = int(p.s) - 1 - p.pad_w;
    return q;
}

}  // namespace

int dgrad_stream_splits(const Prob& p) {
    if (p.stride != 1 || p.groups != 1 || p.pad_h > p.r - 1 || p.pad_w > p.s - 1) return 0;
    return fwd_stream_splits(dgrad_stream_view(p));
}

std::string dgrad_stream_reason(const Prob& p, int splits) {
    if (p.stride != 1) return "the filter-streaming split-K dgrad needs stride 1";
    if (p.groups != 1) return "the filter-streaming split-K dgrad needs groups == 1";
    if (p.pad_h > p.r - 1 || p.pad_w > p.s - 1)
        return "the filter-streaming split-K dgrad needs pad_h <= R-1 and pad_w <= S-1";
    return fwd_stream_reason(dgrad_stream_view(p), splits);
}

bool dgrad_stream_taken(const Prob& p, const Plan& pl) {
    return pl.variant == CNHWC_VAR_DGRAD_SPLITK && pl.split_c > 1 && pl.tune == 0 &&
           dgrad_stream_reason(p, pl.split_c).empty();
}

int launch_dgrad_stream(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx, void* ws,
                        hipStream_t st) {
    const Prob q = dgrad_stream_view(p);
    StreamFwdArgs a{};
    size_t lds;
    if (!stream_geometry(q, pl.split_c, &a, &lds)) return CNHWC_UNSUPPORTED;
    a.x = dy; a.w = w; a.ws = static_cast<float*>(ws);
    a.x_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * p.c * 2);
    a.ws_bytes = uint32_t(int64_t(a.splits) * a.M * q.k * 4);
    a.wchunk_bytes = uint32_t(kSCK * p.r * p.s * p.c * 2);
    const int blocks = a.nblocks;
    const int rc = p.dtype == CNHWC_BF16 ? launch_taps<BF16, true>(int(p.r * p.s), a, lds, blocks, st)
                                         : launch_taps<F16, true>(int(p.r * p.s), a, lds, blocks, st);
    if (rc != CNHWC_OK) return rc;
    return launch_split_reduce(q, a.splits, ws, dx, st);
}

}  // namespace cnhwc
