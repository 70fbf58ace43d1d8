// Depthwise backward-data convolution (groups = C = K) on the vector ALUs,
// in the two forms of "feat(rocke): channel-packed and large-filter depthwise
// dgrad":
//
//  * dw_stream (row streaming, small filters, stride 1 or 2): every lane owns
//    `cpl` adjacent channels of a strip of TW output columns and streams the dY
//    rows of a TH-row band through registers.  Each dY row feeds the dX rows it
//    touches; a dX row is rounded and stored as soon as no later dY row reaches
//    it, so only about R + stride rows of accumulators are live at once (the
//    loop is fully unrolled and the register allocator recycles the flushed
//    rows: the circular accumulator slots of the pages, kept in registers).
//    dY moves as one cpl-wide vector per lane per column, lanes run along the
//    flattened (column strip, channel) index so a wave's loads are contiguous.
//  * dw_rotated (stride 1, filters up to 64 a side, non-square, per-axis
//    padding; the Rotated-filter dgrad section of that page).  At stride 1 the
//    adjoint's index relation dX[h][w] = sum_{r,t} dY[h+pad_h-r][w+pad_w-t] W[r][t]
//    becomes, with r' = R-1-r and t' = S-1-t,
//    dX[h][w] = sum_{r',t'} dY[h-(R-1-pad_h)+r'][w-(S-1-pad_w)+t'] W[R-1-r'][S-1-t'],
//    a plain correlation with the reversed filter whose zero border is
//    R-1-pad_h rows and S-1-pad_w columns.  A block
//    owns a tile of dX rows x columns x 8 channels; the dY window of the tile
//    is staged in LDS as row-pair words (dY[2m][v], dY[2m+1][v]) of one
//    channel, and each lane accumulates 2 rows (an even and an odd one) x 8
//    columns x 2 channels: the even row takes the pair with the filter rows
//    (2k, 2k+1), the odd row the same pair with (2k-1, 2k), so one read pair
//    feeds both rows and no pair is built in the inner loop.  The filter is
//    walked one row pair and 8 columns at a time so only that slice of it sits
//    in registers.  Row pairs whose dY rows are all padding for a wave's rows
//    are skipped.
//
// Arithmetic: pairs of taps along the filter's rows go through one
// v_dot2_f32_{f16,bf16} (two products of the 16-bit inputs added to an fp32
// accumulator), so each lane-op does two multiply-adds without packed-fp32
// instructions; each output is rounded once (RNE) to fp16/bf16.
#include "device.h"
#include "internal.h"

#include <algorithm>
#include <string>

namespace cnhwc {
namespace {

// ============================ row streaming =================================

struct StreamArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, Ho, Wo, pad_h, pad_w;
    int ncv;          // C / cpl
    int nstrips;      // column strips of TW
    int nbands;       // row bands of TH
    int64_t nthreads;
};

template <int CPL>
struct VecT;
template <> struct VecT<1> { using type = unsigned short; };
template <> struct VecT<2> { using type = uint32_t; };
template <> struct VecT<4> { using type = i32x2; };
template <> struct VecT<8> { using type = i32x4; };

template <int CPL>
__device__ inline typename VecT<CPL>::type vload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (CPL == 1) return buf_load2(r, off);
    else if constexpr (CPL == 2) return uint32_t(buf_load4(r, off));
    else if constexpr (CPL == 4) return buf_load8(r, off);
    else return buf_load16(r, off);
}

// 16-bit word j of a cpl-wide vector
template <int CPL>
__device__ inline uint32_t word_of(const typename VecT<CPL>::type& v, int d) {
    if constexpr (CPL == 1) return uint32_t(v);
    else if constexpr (CPL == 2) return v;
    else return uint32_t(v[d]);
}

template <typename T, int R, int S, int ST, int CPL, int TW, int TH>
__global__ __launch_bounds__(256, 2) void dw_stream_kernel(const StreamArgs a) {
    // leaders: filter rows r with (r mod 2*ST) < ST; each pairs with r + ST
    constexpr int NL = (R / (2 * ST)) * ST + ((R % (2 * ST)) < ST ? (R % (2 * ST)) : ST);
    constexpr int VOFF = (S - 1) / ST;               // dY columns left of the strip
    constexpr int NV = (TW - 1) / ST + VOFF + 1;     // dY columns per strip
    constexpr int UL0 = -((R - 1) / ST);             // first pair step (relative)
    constexpr int UL1 = (TH - 1) / ST;               // last pair step
    constexpr int ND = CPL > 1 ? CPL / 2 : 1;        // 32-bit words per vector
    using V = typename VecT<CPL>::type;

    // each XCD (blockIdx % 8) takes a contiguous run of blocks: neighbouring
    // bands of a strip, which read the same halo rows of dY, share its L2
    int bid = blockIdx.x;
    {
        const int q = int(gridDim.x >> 3), rr = int(gridDim.x & 7), x = bid & 7;
        bid = x * q + min(x, rr) + (bid >> 3);
    }
    const int64_t gid = int64_t(bid) * blockDim.x + threadIdx.x;
    if (gid >= a.nthreads) return;
    const int cv = int(gid % a.ncv);
    int64_t rest = gid / a.ncv;
    const int band = int(rest % a.nbands);
    rest /= a.nbands;
    const int strip = int(rest % a.nstrips);
    const int n = int(rest / a.nstrips);
    const int c0 = cv * CPL;

    // tile origin aligned so (h0 + pad_h) and (w0 + pad_w) are multiples of ST
    const int h0 = band * TH - (ST > 1 ? (a.pad_h % ST) : 0);
    const int w0 = strip * TW - (ST > 1 ? (a.pad_w % ST) : 0);
    const int ub = (h0 + a.pad_h) / ST;
    const int vb = (w0 + a.pad_w) / ST - VOFF;

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // weight pairs (W[c][r][t], W[c][r+ST][t]) per leader r, tap t, channel
    uint32_t wp[NL][S][CPL];
    if constexpr (CPL >= 2) {
        // the lane's CPL filters are one contiguous run of CPL*R*S elements
        // starting at an even element (c0 is a multiple of CPL): dword loads,
        // taps picked out at compile-time positions
        constexpr int NWD = CPL * R * S / 2;
        uint32_t fw[NWD];
        const uint32_t base = uint32_t(c0) * (R * S) * 2u;
#pragma unroll
        for (int k = 0; k < NWD; ++k) fw[k] = uint32_t(buf_load4(rw, base + 4u * k));
        auto elem = [&](int f) -> uint32_t { return (fw[f >> 1] >> ((f & 1) * 16)) & 0xffffu; };
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = (i / ST) * 2 * ST + (i % ST);
#pragma unroll
            for (int t = 0; t < S; ++t)
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                    const uint32_t lo = elem(ch * R * S + r * S + t);
                    const uint32_t hi = r + ST < R ? elem(ch * R * S + (r + ST) * S + t) : 0u;
                    wp[i][t][ch] = lo | (hi << 16);
                }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = (i / ST) * 2 * ST + (i % ST);
#pragma unroll
            for (int t = 0; t < S; ++t)
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                    const uint32_t base = uint32_t(c0 + ch) * (R * S);
                    const uint32_t lo = buf_load2(rw, (base + r * S + t) * 2u);
                    const uint32_t hi = r + ST < R ? uint32_t(buf_load2(rw, (base + (r + ST) * S + t) * 2u)) : 0u;
                    wp[i][t][ch] = lo | (hi << 16);
                }
        }
    }

    auto load_row = [&](int u, V (&row)[NV]) {
        const bool uv = u >= 0 && u < a.Ho;
#pragma unroll
        for (int vl = 0; vl < NV; ++vl) {
            const int v = vb + vl;
            uint32_t off = kOob;
            if (uv && v >= 0 && v < a.Wo) off = uint32_t(((n * a.Ho + u) * a.Wo + v) * a.C + c0) * 2u;
            row[vl] = vload<CPL>(rdy, off);
        }
    };

    float acc[TH][TW][CPL];
#pragma unroll
    for (int i = 0; i < TH; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) acc[i][j][ch] = 0.f;

    V prev[NV], cur[NV];
    load_row(ub + UL0 - 1, prev);
#pragma unroll
    for (int ul = UL0; ul <= UL1; ++ul) {
        load_row(ub + ul, cur);
        // pairs (dY[u], dY[u-1]) per column and channel
        uint32_t pr[NV][CPL];
#pragma unroll
        for (int vl = 0; vl < NV; ++vl)
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const uint32_t cw = word_of<CPL>(cur[vl], d), pw = word_of<CPL>(prev[vl], d);
                if constexpr (CPL == 1) {
                    pr[vl][0] = (cw & 0xffffu) | (pw << 16);
                } else {
                    pr[vl][2 * d] = pair_lo(cw, pw);
                    pr[vl][2 * d + 1] = pair_hi(cw, pw);
                }
            }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = (i / ST) * 2 * ST + (i % ST);
            const int hl = ST * ul + r;
            if (hl < 0 || hl >= TH) continue;
#pragma unroll
            for (int wl = 0; wl < TW; ++wl)
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    if (((wl - t) % ST + ST) % ST != 0) continue;
                    const int vl = (wl - t) / ST + VOFF - (((wl - t) < 0 && ((wl - t) % ST) != 0) ? 1 : 0);
#pragma unroll
                    for (int ch = 0; ch < CPL; ++ch)
                        acc[hl][wl][ch] = dot2<T>(pr[vl][ch], wp[i][t][ch], acc[hl][wl][ch]);
                }
        }
        // flush the dX rows no later dY row reaches
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int hl = ST * ul + j;
            if (hl < 0 || hl >= TH) continue;
            const int h = h0 + hl;
            if (h < 0 || h >= a.H) continue;
#pragma unroll
            for (int wl = 0; wl < TW; ++wl) {
                const int w = w0 + wl;
                if (w < 0 || w >= a.W) continue;
                const uint32_t off = uint32_t(((n * a.H + h) * a.W + w) * a.C + c0) * 2u;
                if constexpr (CPL == 1) {
                    buf_store2(pack1<T>(acc[hl][wl][0]), rdx, off);
                } else if constexpr (CPL == 2) {
                    buf_store4(int(pack2<T>(acc[hl][wl][0], acc[hl][wl][1])), rdx, off);
                } else if constexpr (CPL == 4) {
                    i32x2 o = {int(pack2<T>(acc[hl][wl][0], acc[hl][wl][1])),
                               int(pack2<T>(acc[hl][wl][2], acc[hl][wl][3]))};
                    buf_store8(o, rdx, off);
                } else {
                    i32x4 o = {int(pack2<T>(acc[hl][wl][0], acc[hl][wl][1])),
                               int(pack2<T>(acc[hl][wl][2], acc[hl][wl][3])),
                               int(pack2<T>(acc[hl][wl][4], acc[hl][wl][5])),
                               int(pack2<T>(acc[hl][wl][6], acc[hl][wl][7]))};
                    buf_store16(o, rdx, off);
                }
            }
        }
#pragma unroll
        for (int vl = 0; vl < NV; ++vl) prev[vl] = cur[vl];
    }
}

// The instance table: filter (R = S), stride, channels per lane, strip width
// and band height.  Register budgets keep every instance free of scratch.
struct StreamCfg {
    int r, st, cpl, tw, th;
};
constexpr StreamCfg kStream[] = {
    {3, 1, 8, 2, 16}, {3, 1, 4, 4, 16}, {3, 1, 2, 4, 16}, {3, 1, 1, 8, 16},
    {5, 1, 4, 2, 16}, {5, 1, 2, 4, 16}, {5, 1, 1, 4, 16},
    {7, 1, 2, 4, 16}, {7, 1, 1, 4, 16},
    {3, 2, 8, 2, 16}, {3, 2, 4, 4, 16}, {3, 2, 2, 4, 16}, {3, 2, 1, 8, 16},
    {5, 2, 4, 2, 16}, {5, 2, 2, 4, 16}, {5, 2, 1, 4, 16},
    {7, 2, 2, 4, 16}, {7, 2, 1, 4, 16},
};

const StreamCfg* find_stream(const Prob& p, int cpl) {
    for (const StreamCfg& c : kStream)
        if (c.r == p.r && c.r == p.s && c.st == p.stride && c.cpl == cpl) return &c;
    return nullptr;
}

template <typename T, int R, int ST, int CPL, int TW, int TH>
void launch_stream_t(const StreamArgs& a, hipStream_t st) {
    const int64_t blocks = (a.nthreads + 255) / 256;
    hipLaunchKernelGGL((dw_stream_kernel<T, R, R, ST, CPL, TW, TH>), dim3(blocks), dim3(256), 0, st, a);
}

template <typename T>
bool dispatch_stream(const StreamCfg& c, const StreamArgs& a, hipStream_t st) {
#define CNHWC_DWS(R_, ST_, CPL_, TW_, TH_)                                                  \
    if (c.r == R_ && c.st == ST_ && c.cpl == CPL_ && c.tw == TW_ && c.th == TH_) {          \
        launch_stream_t<T, R_, ST_, CPL_, TW_, TH_>(a, st);                                 \
        return true;                                                                        \
    }
    CNHWC_DWS(3, 1, 8, 2, 16) CNHWC_DWS(3, 1, 4, 4, 16) CNHWC_DWS(3, 1, 2, 4, 16) CNHWC_DWS(3, 1, 1, 8, 16)
    CNHWC_DWS(5, 1, 4, 2, 16) CNHWC_DWS(5, 1, 2, 4, 16) CNHWC_DWS(5, 1, 1, 4, 16)
    CNHWC_DWS(7, 1, 2, 4, 16) CNHWC_DWS(7, 1, 1, 4, 16)
    CNHWC_DWS(3, 2, 8, 2, 16) CNHWC_DWS(3, 2, 4, 4, 16) CNHWC_DWS(3, 2, 2, 4, 16) CNHWC_DWS(3, 2, 1, 8, 16)
    CNHWC_DWS(5, 2, 4, 2, 16) CNHWC_DWS(5, 2, 2, 4, 16) CNHWC_DWS(5, 2, 1, 4, 16)
    CNHWC_DWS(7, 2, 2, 4, 16) CNHWC_DWS(7, 2, 1, 4, 16)
#undef CNHWC_DWS
    return false;
}

// ============================ LDS-tiled (small filters) =====================
//
// Stride-1 depthwise dgrad for R x S <= 7 x 7 with the dY window of a tile
// staged in LDS.  A block owns 8 x 28 dX pixels x 64 channels: the window (R-1
// rows and S-1 columns of halo) is loaded with 16-byte asynchronous loads
// straight into LDS, 128 bytes per pixel, and the block's weights go to LDS as
// row pairs (over the staged filter).  Each lane then owns 4 x 7 pixels x 2
// channels: it walks the window rows once, makes the vertical pairs
// (dY[u][v], dY[u-1][v]) of its two channels with one byte permute each, and
// feeds every pair to all the outputs and taps that use it
// (dX[h][w] += pair . (W[r][t], W[r+1][t]) with u = h + R - r, v = w + S-1-t in
// window coordinates) -- all indices compile-time, so the inner loop is a
// straight line of dot2 instructions.
constexpr int kTileTWL = 7;                  // lane tile columns
constexpr int kTilePBH = 2, kTilePBW = 4;    // lane tiles per block tile
constexpr int kTileTW = kTileTWL * kTilePBW; // 28
constexpr int kTileCB = 64;                  // channels per block
// lane tile rows
// (2 for 7x7: its 7 x 4 weight pairs and 2 x 7 x 2 accumulators fill the
// register file)
constexpr int tile_thl(int r) { return r >= 7 ? 2 : 4; }
constexpr int tile_th(int r) { return tile_thl(r) * kTilePBH; }

struct TileArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, Ho, Wo, pad_h, pad_w;
    int tiles_h, tiles_w, cblocks;
    int nblocks, remap;
    int flip;          // 1: use the filter rotated by 180 degrees (depthwise forward)
    FastDiv fd_tw, fd_th, fd_cb;   // division by tiles_w, tiles_h, cblocks
};

template <int R, int S>
struct TileGeo {
    static constexpr int NL = (R + 1) / 2;                    // filter row pairs
    static constexpr int THL = tile_thl(R);
    static constexpr int TH = THL * kTilePBH;
    static constexpr int WR = TH + R - 1;                     // window rows
    static constexpr int WC = kTileTW + S - 1;                // window columns
    static constexpr int NPIX = WR * WC;
    static constexpr int WIN_BYTES = (NPIX + 7) / 8 * 1024;   // whole 8-pixel loads
    static constexpr int RAW_BYTES = (kTileCB * R * S * 2 + 1023) / 1024 * 1024;
    static constexpr int LDS = WIN_BYTES + RAW_BYTES;
};

// blocks per CU: 3x3 four (40 KiB of LDS, 100 VGPRs); 5x5 and 7x7 two (their
// 180-230 VGPRs allow no more, whatever the LDS)
constexpr int tile_occupancy(int r) { return r == 3 ? 4 : 2; }

// Accumulates a lane tile (THL rows x kTileTWL columns x 2 channels) from a
// staged window: win points at the lane tile's first window pixel and channel
// pair (window pixels 128 bytes apart, rows kTileTW + S - 1 pixels long).
// Window row ul - 1 of the lane tile is walked at step ul; the pair partner of
// the first row (one row above the window) only ever meets the zero filter row
// R of odd R, so any finite value serves: the first row itself.
template <typename T, int R, int S, int THL>
__device__ __forceinline__ void tile_accumulate(const uint32_t* win, const uint32_t (&wp)[(R + 1) / 2][S][2],
                                                float (&acc)[THL][kTileTWL][2]) {
    constexpr int WC = kTileTW + S - 1;
    constexpr int RV = kTileTWL + S - 1;                      // window columns a lane reads
#pragma unroll
    for (int h = 0; h < THL; ++h)
#pragma unroll
        for (int w = 0; w < kTileTWL; ++w) acc[h][w][0] = acc[h][w][1] = 0.f;
    uint32_t prev[RV], cur[RV];
#pragma unroll
    for (int v = 0; v < RV; ++v) prev[v] = win[v * 32];
#pragma unroll
    for (int ul = 1; ul < THL + R; ++ul) {
#pragma unroll
        for (int v = 0; v < RV; ++v) cur[v] = win[((ul - 1) * WC + v) * 32];
        uint32_t p0[RV], p1[RV];
#pragma unroll
        for (int v = 0; v < RV; ++v) {
            p0[v] = pair_lo(cur[v], prev[v]);   // channel 2cp: (row ul, row ul-1)
            p1[v] = pair_hi(cur[v], prev[v]);   // channel 2cp+1
        }
#pragma unroll
        for (int hl = 0; hl < THL; ++hl) {
            const int r = hl + R - ul;         // first tap row of the pair
            if (r < 0 || r >= R || (r & 1)) continue;
            // tap-outer: consecutive dot2s update different accumulators
#pragma unroll
            for (int t = 0; t < S; ++t) {
                const uint32_t w0 = wp[r / 2][t][0], w1 = wp[r / 2][t][1];
#pragma unroll
                for (int wl = 0; wl < kTileTWL; ++wl) {
                    const int v = wl + S - 1 - t;
                    acc[hl][wl][0] = dot2<T>(p0[v], w0, acc[hl][wl][0]);
                    acc[hl][wl][1] = dot2<T>(p1[v], w1, acc[hl][wl][1]);
                }
            }
        }
#pragma unroll
        for (int v = 0; v < RV; ++v) prev[v] = cur[v];
    }
}

// Stores a lane tile at dX (n, h .., w .., channels c, c + 1): 4 bytes a pixel.
template <typename T, int THL, typename Args>
__device__ __forceinline__ void tile_store(const Args& a, __amdgpu_buffer_rsrc_t rdx,
                                           const float (&acc)[THL][kTileTWL][2], int n, int h0, int w0,
                                           int c) {
    if (c >= a.C) return;
    // offsets step by a pixel (2C bytes) along the row and by a row (2WC)
    const uint32_t pix = uint32_t(a.C) * 2u, row = uint32_t(a.W) * pix;
    uint32_t off0 = uint32_t(((n * a.H + h0) * a.W + w0) * a.C + c) * 2u;
#pragma unroll
    for (int hl = 0; hl < THL; ++hl) {
        uint32_t off = off0;
#pragma unroll
        for (int wl = 0; wl < kTileTWL; ++wl) {
            if (h0 + hl < a.H && w0 + wl < a.W)
                buf_store4(int(pack2<T>(acc[hl][wl][0], acc[hl][wl][1])), rdx, off);
            off += pix;
        }
        off0 += row;
    }
}

template <typename T, int R, int S>
__global__ __launch_bounds__(256, tile_occupancy(R)) void dw_tile_kernel(const TileArgs a) {
    using G = TileGeo<R, S>;
    constexpr int NL = G::NL, WC = G::WC, NPIX = G::NPIX;
    constexpr int kTileTHL = G::THL, kTileTH = G::TH;
    __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS];
    const unsigned short* const raw = reinterpret_cast<const unsigned short*>(lds + G::WIN_BYTES);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Blocks are dealt to the 8 XCDs round-robin; remap so each XCD walks
    // whole (image, channel block) groups in raster order and vertically
    // neighbouring tiles, which share halo rows, meet in the same L2.
    int bid = blockIdx.x;
    if (a.remap) bid = (bid & 7) * (a.nblocks >> 3) + (bid >> 3);
    const int b1 = fdiv(bid, a.fd_tw), b2 = fdiv(b1, a.fd_th), n = fdiv(b2, a.fd_cb);
    const int tw_i = bid - b1 * a.tiles_w, th_i = b1 - b2 * a.tiles_h, cb = b2 - n * a.cblocks;
    const int h0 = th_i * kTileTH, w0 = tw_i * kTileTW, c0 = cb * kTileCB;

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // ---- window: pixel q = (row, col) holds dY(h0 + pad_h - (R-1) + row, w0 + pad_w - (S-1) + col) ----
    // One load instruction stages 8 consecutive pixels of one window row
    // (8 lanes a pixel, 16 bytes each): its row and column group are uniform,
    // so only the lane's column and the range checks are per-lane work.  Lanes
    // past the row's end load nothing (their LDS slots are the next row's).
    {
        constexpr int CG = (WC + 7) / 8;                      // column groups a row
        constexpr int NLD = G::WR * CG;                       // load instructions a block
        const int chunk = lane & 7, lpx = lane >> 3;
        const bool cin = c0 + chunk * 8 < a.C;
        const int u0 = h0 + a.pad_h - (R - 1), v0 = w0 + a.pad_w - (S - 1);
        const int pix_b = a.C * 2;
        const int lane_off = lpx * pix_b + (c0 + chunk * 8) * 2;
#pragma unroll
        for (int i = 0; i < (NLD + 3) / 4; ++i) {
            const int j = wave + 4 * i;
            if (j < NLD) {
                const int r = j / CG, g = j - (j / CG) * CG;
                const int u = u0 + r, col = 8 * g + lpx, v = v0 + col;
                const bool ok = cin && unsigned(u) < unsigned(a.Ho) && unsigned(v) < unsigned(a.Wo);
                const int off = ((n * a.Ho + u) * a.Wo + v0 + 8 * g) * pix_b + lane_off;
                if (col < WC) dma16(rdy, lds + (r * WC + 8 * g) * 128, ok ? uint32_t(off) : kOob, 0);
            }
        }
    }
    // ---- the block's filters: 64 channels x R*S taps, contiguous in W ----
    // (the block's base goes in the lane offset, which the range check covers:
    // the last channel block's rows past C read zeros)
#pragma unroll
    for (int i = 0; i < G::RAW_BYTES / 1024; ++i)
        if ((i & 3) == wave)
            dma16(rw, lds + G::WIN_BYTES + i * 1024, uint32_t(c0 * R * S * 2 + i * 1024 + lane * 16), 0);
    wait_vm<0>();
    __syncthreads();
    const int cp = lane & 31;                                 // channel pair
    const int pb = 2 * wave + (lane >> 5);
    const int lr0 = (pb / kTilePBW) * kTileTHL, lc0 = (pb % kTilePBW) * kTileTWL;

    // ---- weight pairs: word (i, t, ch) = (W[c][2i][t], W[c][2i+1][t]), built
    // in place over the staged filter (every thread first reads the taps of
    // its words, then all write them), then each lane keeps its two channels'
    // words in registers.  The rotated filter of the depthwise forward reads
    // (R-1-r, S-1-t). ----
    // Word e = (i * S + t) * 64 + ch; a thread's words are e = tid + 256 k, so
    // its channel is tid % 64 and (i, t) depend on the wave and k only.
    constexpr int WTS = NL * S * kTileCB;
    constexpr int WPT = (WTS + 255) / 256;                    // words per thread
    static_assert(WTS * 4 <= G::RAW_BYTES, "weight pairs fit over the staged filter");
    static_assert(256 % kTileCB == 0, "a thread keeps one channel");
    const unsigned short* const wch = raw + (tid % kTileCB) * R * S;
    uint32_t word[WPT];
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
        const int it = wave + (256 / kTileCB) * k;            // i * S + t
        word[k] = 0u;
        if (it < NL * S) {
            const int i = it / S, t = it - (it / S) * S;
            auto tap = [&](int r) {
                return a.flip ? uint32_t(wch[(R - 1 - r) * S + (S - 1 - t)]) : uint32_t(wch[r * S + t]);
            };
            const uint32_t lo = tap(2 * i);
            const uint32_t hi = 2 * i + 1 < R ? tap(2 * i + 1) : 0u;
            word[k] = lo | (hi << 16);
        }
    }
    __syncthreads();
    uint32_t* const wts = reinterpret_cast<uint32_t*>(lds + G::WIN_BYTES);
#pragma unroll
    for (int k = 0; k < WPT; ++k)
        if (wave + (256 / kTileCB) * k < NL * S) wts[tid + 256 * k] = word[k];
    __syncthreads();

    uint32_t wp[NL][S][2];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const i32x2 v = *reinterpret_cast<const i32x2*>(wts + (i * S + t) * kTileCB + cp * 2);
            wp[i][t][0] = uint32_t(v[0]);
            wp[i][t][1] = uint32_t(v[1]);
        }

    float acc[kTileTHL][kTileTWL][2];
    tile_accumulate<T, R, S, kTileTHL>(reinterpret_cast<const uint32_t*>(lds) + (lr0 * WC + lc0) * 32 + cp,
                                       wp, acc);
    tile_store<T, kTileTHL>(a, rdx, acc, n, h0 + lr0, w0 + lc0, c0 + 2 * cp);
}

// tile_accumulate over window rows WC pixels apart, with the next window row
// read one step ahead and the steps fenced off from each other in the
// schedule.
template <typename T, int R, int S, int THL, int WC>
__device__ __forceinline__ void tile_accumulate_pf(const uint32_t* win, const uint32_t (&wp)[(R + 1) / 2][S][2],
                                                   float (&acc)[THL][kTileTWL][2]) {
    constexpr int RV = kTileTWL + S - 1;
    constexpr int NU = THL + R - 1;
#pragma unroll
    for (int h = 0; h < THL; ++h)
#pragma unroll
        for (int w = 0; w < kTileTWL; ++w) acc[h][w][0] = acc[h][w][1] = 0.f;
    uint32_t prev[RV], cur[RV];
#pragma unroll
    for (int v = 0; v < RV; ++v) prev[v] = win[v * 32];
#pragma unroll
    for (int v = 0; v < RV; ++v) cur[v] = win[v * 32];
#pragma unroll
    for (int ul = 1; ul <= NU; ++ul) {
        uint32_t nxt[RV];
        if (ul < NU) {
#pragma unroll
            for (int v = 0; v < RV; ++v) nxt[v] = win[(ul * WC + v) * 32];
        }
        uint32_t p0[RV], p1[RV];
#pragma unroll
        for (int v = 0; v < RV; ++v) {
            p0[v] = pair_lo(cur[v], prev[v]);
            p1[v] = pair_hi(cur[v], prev[v]);
        }
#pragma unroll
        for (int hl = 0; hl < THL; ++hl) {
            const int r = hl + R - ul;
            if (r < 0 || r >= R || (r & 1)) continue;
#pragma unroll
            for (int t = 0; t < S; ++t) {
                const uint32_t w0 = wp[r / 2][t][0], w1 = wp[r / 2][t][1];
#pragma unroll
                for (int wl = 0; wl < kTileTWL; ++wl) {
                    const int v = wl + S - 1 - t;
                    acc[hl][wl][0] = dot2<T>(p0[v], w0, acc[hl][wl][0]);
                    acc[hl][wl][1] = dot2<T>(p1[v], w1, acc[hl][wl][1]);
                }
            }
        }
#pragma unroll
        for (int v = 0; v < RV; ++v) prev[v] = cur[v];
        if (ul < NU) {
#pragma unroll
            for (int v = 0; v < RV; ++v) cur[v] = nxt[v];
        }
        // the step's products finish before the next step's reads issue (the
        // compiler otherwise issues every row's reads first and runs out of
        // registers holding them)
#pragma unroll
        for (int hl = 0; hl < THL; ++hl)
#pragma unroll
            for (int wl = 0; wl < kTileTWL; ++wl) asm volatile("" : "+v"(acc[hl][wl][0]), "+v"(acc[hl][wl][1]));
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ============================ LDS-tiled, persistent (7 x 7) ==================
//
// The 7x7 case of the LDS-tiled dgrad with two resident blocks a CU, each
// walking a contiguous run of the tiles of one channel block: the weight
// pairs are built once a block, and while one block waits for its next
// window the other multiplies.  A lane owns 4 x 7 pixels x 2 channels, so
// every window row it reads and pairs feeds twice the outputs of the two-row
// lane tile; a block tile is 8 x 28 pixels x 64 channels.  The products are
// v_dot2 instructions, which a SIMD issues at about one every 6 cycles with
// two waves resident (measured), so the kernel is bound by that issue rate.
constexpr int kPipeTHL = 4;                       // lane tile rows
constexpr int kPipeTH = kPipeTHL * kTilePBH;      // block tile rows
constexpr int kPipeBlocksPerCU = 2;

template <int R, int S>
struct PipeGeo {
    static constexpr int NL = (R + 1) / 2;
    static constexpr int WR = kPipeTH + R - 1;                // window rows
    static constexpr int CG = (kTileTW + S - 1 + 7) / 8;      // 8-pixel column groups a row
    static constexpr int WC = CG * 8;                         // window row pitch (pixels)
    static constexpr int NLD = WR * CG;                       // load instructions a window
    static constexpr int LPW = (NLD + 3) / 4;                 // of them a wave
    // the window, then the slots of the 4 LPW - NLD spare loads
    static constexpr int WIN_BYTES = 4 * LPW * 1024;
    static constexpr int RAW_BYTES = (kTileCB * R * S * 2 + 1023) / 1024 * 1024;
    static constexpr int LDS = WIN_BYTES + RAW_BYTES;   // two blocks fit a CU
};

struct PipeArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, Ho, Wo, pad_h, pad_w;
    int tiles_h, tiles_w;
    int tiles_cb;      // tiles of one channel block: N * tiles_h * tiles_w
    int bq, br;        // blocks a channel block: bq + 1 for the first br, bq for the rest
    int flip;          // 1: use the filter rotated by 180 degrees (depthwise forward)
    FastDiv fd_tw, fd_th;   // division by tiles_w, tiles_h
};

template <typename T, int R, int S>
__global__ __launch_bounds__(256, kPipeBlocksPerCU) void dw_tilep_kernel(const PipeArgs a) {
    using G = PipeGeo<R, S>;
    constexpr int NL = G::NL, WC = G::WC, CG = G::CG, NLD = G::NLD, LPW = G::LPW;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char* const raw_b = lds + G::WIN_BYTES;
    const unsigned short* const raw = reinterpret_cast<const unsigned short*>(raw_b);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // block -> channel block cb (bq or bq + 1 blocks each) and its tiles j,
    // j + nb, j + 2 nb, ...: the nb blocks of a channel block take consecutive
    // tiles at the same time, and each XCD (blockIdx % 8) a contiguous run of
    // blocks, so the tiles that share halo rows and columns are loaded
    // through one L2 at about the same time
    int bid = blockIdx.x;
    {
        const int q = int(gridDim.x >> 3), rr = int(gridDim.x & 7), x = bid & 7;
        bid = x * q + min(x, rr) + (bid >> 3);
    }
    const int big = a.br * (a.bq + 1);
    int cb, j, nb;
    if (bid < big) {
        nb = a.bq + 1;
        cb = bid / nb;
        j = bid - cb * nb;
    } else {
        nb = a.bq;
        const int b = bid - big;
        cb = a.br + b / nb;
        j = b - (b / nb) * nb;
    }
    if (j >= a.tiles_cb) return;   // block-uniform
    const int c0 = cb * kTileCB;

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // tile t of the channel block: image n, rows h0 .., columns w0 .. (raster
    // order within an image, so consecutive tiles share halo columns or rows)
    auto tile_of = [&](int t, int& n, int& h0, int& w0) {
        const int b1 = fdiv(t, a.fd_tw);
        const int tw = t - b1 * a.tiles_w;
        n = fdiv(b1, a.fd_th);
        h0 = (b1 - n * a.tiles_h) * kPipeTH;
        w0 = tw * kTileTW;
    };
    // Window load i of this wave (instruction wave + 4 i: window row r, pixels
    // 8 g .. 8 g + 7, 8 lanes a pixel) of the tile at (n, h0, w0); window pixel
    // (row, col) holds dY(h0 + pad_h - (R-1) + row, w0 + pad_w - (S-1) + col),
    // zero outside the image.  The row pitch is whole 8-pixel groups, so no
    // lane's slot belongs to another row and nothing here branches per lane
    // (divergent branches in the unrolled tile loop cost the register file).
    const int chunk = lane & 7, lpx = lane >> 3;
    const bool cin = c0 + chunk * 8 < a.C;
    const int pix_b = a.C * 2;
    const int lane_off = lpx * pix_b + (c0 + chunk * 8) * 2;
    // Every wave issues LPW loads; the spare ones read zeros into slots
    // nothing reads, so no branch splits the tile loop.
    auto issue = [&](int i, int n, int h0, int w0) {
        // the wave index laundered per call: the scalar terms of the 4 x
        // LPW loads are not hoisted out of the tile loop (register pressure)
        int wv = wave;
        asm volatile("" : "+s"(wv));
        const int jj = wv + 4 * i;
        const int r = jj / CG, g = jj - (jj / CG) * CG;
        const int u = h0 + a.pad_h - (R - 1) + r;
        const int v00 = w0 + a.pad_w - (S - 1) + 8 * g;
        const bool ok = jj < NLD && cin && unsigned(u) < unsigned(a.Ho) && unsigned(v00 + lpx) < unsigned(a.Wo);
        const int off = ((n * a.Ho + u) * a.Wo + v00) * pix_b + lane_off;
        // LDS slot (r * WC + 8 g) * 128 = jj * 1024 (the row pitch is CG groups)
        dma16(rdy, lds + jj * 1024, ok ? uint32_t(off) : kOob, 0);
    };

    // ---- the block's filters (64 channels x R*S taps, contiguous in W; rows
    // past C read zeros) and the first tile's window ----
    int n, h0, w0;
    tile_of(j, n, h0, w0);
#pragma unroll
    for (int i = 0; i < G::RAW_BYTES / 1024; ++i)
        if ((i & 3) == wave) dma16(rw, raw_b + i * 1024, uint32_t(c0 * R * S * 2 + i * 1024 + lane * 16), 0);
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue(i, n, h0, w0);
    wait_vm<0>();
    __syncthreads();

    // ---- weight pairs, as in the one-tile kernel: word (i, t, ch) =
    // (W[c][2i][t], W[c][2i+1][t]) built in place over the staged filter ----
    constexpr int WTS = NL * S * kTileCB;
    constexpr int WPT = (WTS + 255) / 256;
    static_assert(WTS * 4 <= G::RAW_BYTES, "weight pairs fit over the staged filter");
    const unsigned short* const wch = raw + (tid % kTileCB) * R * S;
    uint32_t word[WPT];
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
        const int it = wave + (256 / kTileCB) * k;
        word[k] = 0u;
        if (it < NL * S) {
            const int i = it / S, t = it - (it / S) * S;
            auto tap = [&](int r) {
                return a.flip ? uint32_t(wch[(R - 1 - r) * S + (S - 1 - t)]) : uint32_t(wch[r * S + t]);
            };
            const uint32_t lo = tap(2 * i);
            const uint32_t hi = 2 * i + 1 < R ? tap(2 * i + 1) : 0u;
            word[k] = lo | (hi << 16);
        }
    }
    __syncthreads();
    uint32_t* const wts = reinterpret_cast<uint32_t*>(raw_b);
#pragma unroll
    for (int k = 0; k < WPT; ++k)
        if (wave + (256 / kTileCB) * k < NL * S) wts[tid + 256 * k] = word[k];
    __syncthreads();
    const int cp = lane & 31;
    const int pb = 2 * wave + (lane >> 5);
    const int lr0 = (pb / kTilePBW) * kPipeTHL, lc0 = (pb % kTilePBW) * kTileTWL;
    uint32_t wp[NL][S][2];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const i32x2 v = *reinterpret_cast<const i32x2*>(wts + (i * S + t) * kTileCB + cp * 2);
            wp[i][t][0] = uint32_t(v[0]);
            wp[i][t][1] = uint32_t(v[1]);
        }

    // ---- the run: multiply tile t, let every wave finish reading the window,
    // start the next window's loads over it, store tile t, and wait for the
    // loads (the other block on the CU multiplies meanwhile) ----
#pragma unroll 1
    for (int t = j; t < a.tiles_cb; t += nb) {
        const bool more = t + nb < a.tiles_cb;
        int n1 = n, h1 = h0, w1 = w0;
        if (more) tile_of(t + nb, n1, h1, w1);
        const uint32_t* const win = reinterpret_cast<const uint32_t*>(lds) + (lr0 * WC + lc0) * 32 + cp;
        float acc[kPipeTHL][kTileTWL][2];
        tile_accumulate_pf<T, R, S, kPipeTHL, WC>(win, wp, acc);
        // the sums are complete here: otherwise the compiler sinks the last
        // steps' products past the barrier among the stores, where they
        // overflow the register file
#pragma unroll
        for (int hl = 0; hl < kPipeTHL; ++hl)
#pragma unroll
            for (int wl = 0; wl < kTileTWL; ++wl) asm volatile("" : "+v"(acc[hl][wl][0]), "+v"(acc[hl][wl][1]));
        __syncthreads();
        if (more) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) issue(i, n1, h1, w1);
        }
        // stores of pixels outside dX (or channels past C) are dropped by the
        // buffer range check
        {
            const int c = c0 + 2 * cp, hh = h0 + lr0, ww = w0 + lc0;
            const uint32_t pix = uint32_t(a.C) * 2u;
            const uint32_t off0 = uint32_t(((n * a.H + hh) * a.W + ww) * a.C + c) * 2u;
#pragma unroll
            for (int hl = 0; hl < kPipeTHL; ++hl)
#pragma unroll
                for (int wl = 0; wl < kTileTWL; ++wl) {
                    const bool in = c < a.C && hh + hl < a.H && ww + wl < a.W;
                    const uint32_t off = off0 + uint32_t(hl * a.W + wl) * pix;
                    buf_store4(int(pack2<T>(acc[hl][wl][0], acc[hl][wl][1])), rdx, in ? off : kOob);
                }
        }
        wait_vm<0>();
        __syncthreads();
        n = n1; h0 = h1; w0 = w1;
    }
}

// ============================ rotated filter ================================

constexpr int kRotCB = 8;      // channels per block
constexpr int kRotTHT = 2;     // output rows per lane
constexpr int kRotTWT = 8;     // output columns per lane
constexpr int kRotTB = 8;      // filter columns per register slice (wide filters)
constexpr int kRotPadCols = 8; // window columns between LDS pad words
constexpr int kRotMaxF = 64;   // largest filter side
constexpr int kRotSplit = 2;   // lane groups splitting the filter steps of a tile

struct RotArgs {
    const void* dy;
    const void* w;
    void* dx;
    uint32_t dy_bytes, w_bytes, dx_bytes;
    int N, H, W, C, Ho, Wo, R, S;
    int ph2, pw2;          // padding of the correlation (dgrad: R-1-pad_h, S-1-pad_w)
    int rot;               // 1: correlate with the filter rotated by 180 degrees (dgrad)
    int OHB, OWB;          // output tile of a block
    int IHB, IWB;          // staged dY window (rows: 2 x pair rows; columns padded to slices)
    int rpairs, tslices;   // R/2 + 1 filter row pairs, ceil(S/TB) column slices
    int tiles_h, tiles_w, cblocks;
    int row_dw;            // LDS words of one pair row
};

// Block: 256 lanes = 4 channel pairs x 4 column groups (8 columns) x 16 row
// groups (2 rows): a 32 x 32 x 8 output tile.  TB: filter columns per
// register slice -- 8 for filters wider than 7 columns, else the filter
// width itself (one slice, no zero columns multiplied).
template <typename T, int SPLIT, int TB>
__global__ __launch_bounds__(256 * SPLIT, 1) void dw_rotated_kernel(const RotArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    constexpr int NT = 256 * SPLIT;
    const int tid = threadIdx.x;
    const int lt = tid & 255, grp = tid >> 8;      // lane role within its group; tap group
    const int cp = lt & 3, cg = (lt >> 2) & 3, rg = lt >> 4;
    // Blocks are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8); remap
    // so each XCD takes a contiguous run of the order below, channel block
    // fastest: the blocks whose 16-byte channel slices share a pixel's
    // 128-byte lines then share one L2, which fetches those dY lines once and
    // merges their dX writes into whole lines
    int bid = blockIdx.x;
    {
        const int q = int(gridDim.x >> 3), rr = int(gridDim.x & 7), x = bid & 7;
        bid = x * q + min(x, rr) + (bid >> 3);
    }
    const int cb = bid % a.cblocks;
    bid /= a.cblocks;
    const int tw_ = bid % a.tiles_w;
    bid /= a.tiles_w;
    const int th_ = bid % a.tiles_h;
    const int n = bid / a.tiles_h;
    const int h0 = th_ * a.OHB, w0 = tw_ * a.OWB, c0 = cb * kRotCB;

    const __amdgpu_buffer_rsrc_t rdy = make_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w_bytes);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(a.dx, a.dx_bytes);

    // The dY window is staged as row-pair words: pair row m, column v holds
    // for each of the 8 channels (dY(h0 - ph2 + 2m, w0 - pw2 + v), the row
    // below) in one word.  Layout [m][v][8 channels] with 8 pad words after
    // every 8 columns and a pair-row stride of a.row_dw words (= 32 mod 64):
    // a 64-bit read of 32 lanes (4 channel pairs x 4 column groups 8 columns
    // apart x 2 row groups one pair row apart) then covers the 64 banks once.
    // A lane loads a batch of its window positions before writing any.
    uint32_t* win = smem;
    const int npp = (a.IHB / 2) * a.IWB;
    constexpr int kWinBatch = 4;
    i32x4 top[kWinBatch], bot[kWinBatch];
    auto win_load = [&](int q0) {
#pragma unroll
        for (int b = 0; b < kWinBatch; ++b) {
            const int q = q0 + b * NT;
            const int m = q / a.IWB, iw = q - m * a.IWB;
            const int u = h0 - a.ph2 + 2 * m, v = w0 - a.pw2 + iw;
            const bool vin = q < npp && v >= 0 && v < a.Wo;
            const uint32_t off = uint32_t(((n * a.Ho + u) * a.Wo + v) * a.C + c0) * 2u;
            top[b] = buf_load16(rdy, vin && u >= 0 && u < a.Ho ? off : kOob);
            bot[b] = buf_load16(rdy, vin && u + 1 >= 0 && u + 1 < a.Ho ? off + uint32_t(a.Wo * a.C * 2) : kOob);
        }
    };
    auto win_write = [&](int q0) {
#pragma unroll
        for (int b = 0; b < kWinBatch; ++b) {
            const int q = q0 + b * NT;
            const int m = q / a.IWB, iw = q - m * a.IWB;
            if (q < npp) {
                i32x4 lo, hi;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    lo[2 * j] = int(pair_lo(uint32_t(top[b][j]), uint32_t(bot[b][j])));
                    lo[2 * j + 1] = int(pair_hi(uint32_t(top[b][j]), uint32_t(bot[b][j])));
                    hi[2 * j] = int(pair_lo(uint32_t(top[b][j + 2]), uint32_t(bot[b][j + 2])));
                    hi[2 * j + 1] = int(pair_hi(uint32_t(top[b][j + 2]), uint32_t(bot[b][j + 2])));
                }
                i32x4* dst = reinterpret_cast<i32x4*>(win + m * a.row_dw + iw * 8 + (iw / kRotPadCols) * 8);
                dst[0] = lo;
                dst[1] = hi;
            }
        }
    };

    // ---- the block's filter slice (8 channels x R x S halves, contiguous in
    // W: R*S 16-byte pieces) and the window's first batch go out together;
    // the slice lands in the window's LDS, where the pair words are built
    // from it before the window overwrites it (the window region holds at
    // least 18 R S bytes, the slice 16 R S) ----
    constexpr int kRawPT = (kRotMaxF * kRotMaxF + NT - 1) / NT;
    const int nraw = a.R * a.S;
    const int nraw_pt = (nraw + NT - 1) / NT;
    i32x4 rawv[kRawPT];
#pragma unroll
    for (int k = 0; k < kRawPT; ++k) {
        const int q = tid + k * NT;
        if (k < nraw_pt) rawv[k] = buf_load16(rw, q < nraw ? uint32_t(c0 * nraw * 2 + q * 16) : kOob);
    }
    win_load(tid);
    wait_vm<2 * kWinBatch>();   // the slice (the window batch stays in flight)
#pragma unroll
    for (int k = 0; k < kRawPT; ++k) {
        const int q = tid + k * NT;
        if (k < nraw_pt && q < nraw) reinterpret_cast<i32x4*>(win)[q] = rawv[k];
    }
    __syncthreads();
    // ---- filter pair words: even set [k][t][8 channels] = (W'(2k, t),
    // W'(2k+1, t)), odd set = (W'(2k-1, t), W'(2k, t)), with W' the
    // correlation's filter (rotated for the dgrad), zero outside it ----
    const unsigned short* raw = reinterpret_cast<const unsigned short*>(win);
    uint32_t* wpe = smem + (a.IHB / 2) * a.row_dw;
    const int tpad = a.tslices * TB;
    const int nwp = a.rpairs * tpad * kRotCB;
    uint32_t* wpo = wpe + nwp;
    for (int q = tid; q < nwp; q += NT) {
        const int ch = q % kRotCB;
        const int t = (q / kRotCB) % tpad;
        const int k = q / (kRotCB * tpad);
        auto tap = [&](int r) -> uint32_t {
            if (t >= a.S || r < 0 || r >= a.R) return 0u;
            const int e = a.rot ? (a.R - 1 - r) * a.S + (a.S - 1 - t) : r * a.S + t;
            return raw[ch * nraw + e];
        };
        const uint32_t t0 = tap(2 * k - 1), t1 = tap(2 * k), t2 = tap(2 * k + 1);
        wpe[q] = t1 | (t2 << 16);
        wpo[q] = t0 | (t1 << 16);
    }
    __syncthreads();   // the slice is read: the window goes over it
    wait_vm<0>();
    win_write(tid);
    for (int q0 = tid + kWinBatch * NT; q0 < npp; q0 += kWinBatch * NT) {
        win_load(q0);
        wait_vm<0>();
        win_write(q0);
    }
    __syncthreads();

    float acc[kRotTHT][kRotTWT][2];
#pragma unroll
    for (int i = 0; i < kRotTHT; ++i)
#pragma unroll
        for (int j = 0; j < kRotTWT; ++j) acc[i][j][0] = acc[i][j][1] = 0.f;

    // rows of this wave: 4 row groups x 2 rows; pair k reads dY rows
    // base + 2k .. base + 2k + 7 over the wave: skip the pairs that only
    // meet padding
    const int wave_row0 = (rg & ~3) * kRotTHT;     // first tile row of the wave
    int rp_lo = 0, rp_hi = a.rpairs;
    {
        const int base = h0 + wave_row0 - a.ph2;
        while (rp_lo < rp_hi && base + 2 * rp_lo + 7 < 0) ++rp_lo;
        while (rp_hi > rp_lo && base + 2 * (rp_hi - 1) >= a.Ho) --rp_hi;
    }
    int ts_lo = 0, ts_hi = a.tslices;
    {
        const int base = w0 - a.pw2;
        while (ts_lo < ts_hi && base + a.OWB - 1 + (ts_lo + 1) * TB - 1 < 0) ++ts_lo;
        while (ts_hi > ts_lo && base + (ts_hi - 1) * TB >= a.Wo) --ts_hi;
    }
    const int orow = rg * kRotTHT, ocol = cg * kRotTWT;
    // The (row pair, column slice) steps are software-pipelined: the LDS reads
    // of the next step (one pair row x 15 columns, 8 even and 8 odd filter
    // pair words) are issued before the dot2s of the current one.
    constexpr int NV = kRotTWT + TB - 1;
    static_assert(TB == kRotTB || TB < kRotPadCols, "a narrow slice is the only one: it starts on a pad group");
    struct Frag {
        uint32_t x[NV][2];
        uint32_t we[TB][2], wo[TB][2];
    };
    // SPLIT groups of 256 lanes compute the same outputs over disjoint runs
    // of the flattened (row pair, column slice) steps; their fp32 sums are
    // added at the end in group order
    const int nts = ts_hi - ts_lo;
    const int total = (rp_hi - rp_lo) * nts;
    const int it_lo = grp * total / SPLIT, it_hi = (grp + 1) * total / SPLIT;
    int lrp = rp_lo + (nts > 0 ? it_lo / nts : 0), lts = ts_lo + (nts > 0 ? it_lo % nts : 0);   // load cursor
    auto load = [&](Frag& f) {
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int wi = (lrp * tpad + lts * TB + t) * kRotCB + cp * 2;
            const i32x2 ve = *reinterpret_cast<const i32x2*>(wpe + wi);
            const i32x2 vo = *reinterpret_cast<const i32x2*>(wpo + wi);
            f.we[t][0] = uint32_t(ve[0]);
            f.we[t][1] = uint32_t(ve[1]);
            f.wo[t][0] = uint32_t(vo[0]);
            f.wo[t][1] = uint32_t(vo[1]);
        }
        // the slice starts on an 8-column boundary, so column vl of it carries
        // (vl >> 3) more pad groups than the first
        const int iw0 = ocol + lts * TB;
        const uint32_t* r0 = win + (rg + lrp) * a.row_dw + iw0 * 8 + (iw0 >> 3) * 8 + cp * 2;
#pragma unroll
        for (int vl = 0; vl < NV; ++vl) {
            const i32x2 v = *reinterpret_cast<const i32x2*>(r0 + vl * 8 + (vl >> 3) * 8);
            f.x[vl][0] = uint32_t(v[0]);
            f.x[vl][1] = uint32_t(v[1]);
        }
        ++lts;
        const bool wrap = lts >= ts_hi;
        lts = wrap ? ts_lo : lts;
        lrp += wrap ? 1 : 0;
    };
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < kRotTWT; ++j)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    acc[0][j][c] = dot2<T>(f.x[j + t][c], f.we[t][c], acc[0][j][c]);
                    acc[1][j][c] = dot2<T>(f.x[j + t][c], f.wo[t][c], acc[1][j][c]);
                }
    };
    Frag fa, fb;
    if (it_lo < it_hi) load(fa);
#pragma unroll 1
    for (int it = it_lo; it < it_hi; it += 2) {
        if (it + 1 < it_hi) load(fb);
        compute(fa);
        if (it + 1 < it_hi) {
            if (it + 2 < it_hi) load(fa);
            compute(fb);
        }
    }
    if constexpr (SPLIT > 1) {
        // groups 1.. park their sums in LDS (the window is no longer read);
        // group 0 adds them in group order and stores
        __syncthreads();
        float* part = reinterpret_cast<float*>(smem);
        constexpr int NA = kRotTHT * kRotTWT * 2;
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < kRotTHT; ++i)
#pragma unroll
                for (int j = 0; j < kRotTWT; ++j)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        part[((grp - 1) * NA + (i * kRotTWT + j) * 2 + c) * 256 + lt] = acc[i][j][c];
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll 1
        for (int g2 = 1; g2 < SPLIT; ++g2)
#pragma unroll
            for (int i = 0; i < kRotTHT; ++i)
#pragma unroll
                for (int j = 0; j < kRotTWT; ++j)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        acc[i][j][c] += part[((g2 - 1) * NA + (i * kRotTWT + j) * 2 + c) * 256 + lt];
    }
    // ---- store: 2 channels per lane ----
#pragma unroll
    for (int i = 0; i < kRotTHT; ++i) {
        const int h = h0 + orow + i;
        if (orow + i >= a.OHB || h >= a.H) continue;
#pragma unroll
        for (int j = 0; j < kRotTWT; ++j) {
            const int w = w0 + ocol + j;
            if (ocol + j >= a.OWB || w >= a.W) continue;
            buf_store4(int(pack2<T>(acc[i][j][0], acc[i][j][1])), rdx,
                       uint32_t(((n * a.H + h) * a.W + w) * a.C + c0 + cp * 2) * 2u);
        }
    }
}

// Filter columns per register slice: the filter width itself up to 7 (one
// slice, no zero columns), else 8-column slices.
int rot_tb(const Prob& p) { return p.s < kRotTB ? int(p.s) : kRotTB; }

bool rot_geometry(const Prob& p, int tb, RotArgs* a, size_t* lds) {
    a->OHB = int(std::min<int64_t>(32, p.h));
    a->OWB = int(std::min<int64_t>(32, p.w));
    a->rpairs = int(p.r / 2 + 1);   // even rows use taps 2k, 2k+1; odd rows 2k-1, 2k
    a->tslices = int((p.s + tb - 1) / tb);
    // rows: tile rows + 2*rpairs (pair k of row group g is pair row g + k);
    // columns: tile + padded slices
    a->IHB = 32 + 2 * a->rpairs;
    a->IWB = 32 + a->tslices * tb;
    // 8 words a column, 8 pad words after every 8 columns, stride = 32 mod 64
    const int base = a->IWB * 8 + (a->IWB / kRotPadCols) * 8;
    a->row_dw = base + ((32 - base % 64) + 64) % 64;
    const size_t win = size_t(a->IHB / 2) * a->row_dw * 4;
    const size_t wts = 2 * size_t(a->rpairs) * a->tslices * tb * kRotCB * 4;
    // the tap groups' partial sums reuse the window's LDS at the end
    const size_t parts = size_t(kRotSplit - 1) * 256 * kRotTHT * kRotTWT * 2 * 4;
    *lds = std::max(win + wts, parts);
    return win + wts <= 160 * 1024;
}

}  // namespace

// ---------------------------------------------------------------------------

int dw_stream_best_cpl(const Prob& p) {
    // two channels per lane measured fastest on MI355X for 3x3 and 7x7 (more
    // lanes in flight beat wider vectors); then wider, then one
    static const int order[] = {2, 4, 8, 1};
    for (int c : order)
        if (p.c % c == 0 && find_stream(p, c)) return c;
    return 0;
}

std::string dw_stream_reason(const Prob& p, int cpl) {
    if (!(p.groups == p.c && p.groups == p.k)) return "depthwise kernels need groups == C == K";
    if (cpl != 1 && cpl != 2 && cpl != 4 && cpl != 8) return "cpl must be 1, 2, 4 or 8";
    if (p.c % cpl != 0) return "channels must be a multiple of cpl";
    if (p.r != p.s) return "row-streaming instances are square filters";
    if (p.stride > 2) return "row streaming supports stride 1 or 2";
    if (!find_stream(p, cpl))
        return "no row-streaming instance for filter " + std::to_string(p.r) + " stride " +
               std::to_string(p.stride) + " cpl " + std::to_string(cpl) +
               " (register budget: filter <= 7; cpl 8 only at 3x3, cpl 4 up to 5x5)";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.k > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    return "";
}

// 7x7 problems (in dgrad terms) run on the persistent kernel unless tune 1
bool dw_tiled_persist_applies(const Prob& p, int tune) { return p.r == 7 && p.s == 7 && tune != 1; }

std::string dw_tiled_reason(const Prob& p) {
    if (!(p.groups == p.c && p.groups == p.k)) return "depthwise kernels need groups == C == K";
    if (p.stride != 1) return "the LDS-tiled depthwise dgrad needs stride 1";
    if (p.r != p.s || (p.r != 3 && p.r != 5 && p.r != 7))
        return "the LDS-tiled depthwise dgrad has 3x3, 5x5 and 7x7 instances";
    if (p.c % 8 != 0) return "the LDS-tiled depthwise dgrad needs C a multiple of 8";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.c > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    return "";
}

std::string dw_rotated_reason(const Prob& p) {
    if (!(p.groups == p.c && p.groups == p.k)) return "depthwise kernels need groups == C == K";
    if (p.stride != 1) return "the rotated-filter dgrad needs stride 1";
    if (p.r > kRotMaxF || p.s > kRotMaxF) return "the rotated-filter dgrad takes filters up to 64 a side";
    if (p.pad_h > p.r - 1 || p.pad_w > p.s - 1)
        return "the rotated-filter dgrad needs pad_h <= R-1 and pad_w <= S-1";
    if (p.c % kRotCB != 0) return "the rotated-filter dgrad needs C a multiple of 8";
    RotArgs a{};
    size_t lds;
    if (!rot_geometry(p, kRotTB, &a, &lds)) return "staged dY window exceeds LDS";
    if (p.h * p.w * p.c > (int64_t(1) << 30) || p.ho * p.wo * p.k > (int64_t(1) << 30))
        return "one image exceeds the 32-bit element range";
    return "";
}

int launch_dgrad_dw_stream(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                           hipStream_t st) {
    const StreamCfg* c = find_stream(p, pl.cpl);
    if (!c) return CNHWC_UNSUPPORTED;
    StreamArgs a{};
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.Ho = int(p.ho); a.Wo = int(p.wo);
    a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.ncv = int(p.c / c->cpl);
    const int st_ = p.stride;
    const int wext = int(p.w) + (st_ > 1 ? p.pad_w % st_ : 0);
    const int hext = int(p.h) + (st_ > 1 ? p.pad_h % st_ : 0);
    a.nstrips = (wext + c->tw - 1) / c->tw;
    a.nbands = (hext + c->th - 1) / c->th;
    a.nthreads = int64_t(a.N) * a.nstrips * a.nbands * a.ncv;
    const bool ok = p.dtype == CNHWC_BF16 ? dispatch_stream<BF16>(*c, a, st) : dispatch_stream<F16>(*c, a, st);
    return ok ? CNHWC_OK : CNHWC_UNSUPPORTED;
}

namespace {
template <typename T>
int launch_tile_t(const Prob& p, const TileArgs& a, int blocks, hipStream_t st) {
    switch (p.r) {
    case 3: hipLaunchKernelGGL((dw_tile_kernel<T, 3, 3>), dim3(blocks), dim3(256), 0, st, a); return CNHWC_OK;
    case 5: hipLaunchKernelGGL((dw_tile_kernel<T, 5, 5>), dim3(blocks), dim3(256), 0, st, a); return CNHWC_OK;
    case 7: hipLaunchKernelGGL((dw_tile_kernel<T, 7, 7>), dim3(blocks), dim3(256), 0, st, a); return CNHWC_OK;
    default: return CNHWC_UNSUPPORTED;
    }
}
}  // namespace

namespace {

// Depthwise forward (stride 1) through the dgrad kernels: y is x correlated
// with the filter at padding pad, which is the dgrad correlation of x (as dY,
// extents H x W) at padding R-1-pad with the filter rotated by 180 degrees --
// the rotation identity of "Depthwise kernels" (Rotated-filter dgrad) read in
// the other direction.  The swapped problem is what the dgrad launchers take.
Prob fwd_as_dgrad(const Prob& p) {
    Prob q = p;
    q.h = p.ho; q.w = p.wo; q.ho = p.h; q.wo = p.w;
    q.pad_h = int(p.r) - 1 - p.pad_h;
    q.pad_w = int(p.s) - 1 - p.pad_w;
    return q;
}

template <typename T>
int launch_tilep_t(const PipeArgs& a, int blocks, hipStream_t st) {
    auto kern = dw_tilep_kernel<T, 7, 7>;
    constexpr size_t lds = PipeGeo<7, 7>::LDS;
    static bool attr_set = false;   // per instance; idempotent if raced
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(lds)) != hipSuccess)
            return CNHWC_HIP_ERROR;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, st, a);
    return CNHWC_OK;
}

// The persistent 7x7 kernel: two blocks a CU (more when there are more channel
// blocks than that), each channel block's tiles dealt to its blocks in turn
// (block j of nb takes tiles j, j + nb, ...).
int launch_tiled_persistent(const Prob& p, int flip, const void* dy, const void* w, void* dx,
                            hipStream_t st) {
    PipeArgs a{};
    a.flip = flip;
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.Ho = int(p.ho); a.Wo = int(p.wo);
    a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    a.tiles_h = int((p.h + kPipeTH - 1) / kPipeTH);
    a.tiles_w = int((p.w + kTileTW - 1) / kTileTW);
    const int64_t cblocks = (p.c + kTileCB - 1) / kTileCB;
    const int64_t tiles_cb = int64_t(a.N) * a.tiles_h * a.tiles_w;
    const int64_t blocks =
        std::max<int64_t>(cblocks, std::min<int64_t>(kPipeBlocksPerCU * kNumCUs, tiles_cb * cblocks));
    a.tiles_cb = int(tiles_cb);
    a.bq = int(blocks / cblocks);
    a.br = int(blocks % cblocks);
    a.fd_tw = make_fastdiv(uint32_t(a.tiles_w));
    a.fd_th = make_fastdiv(uint32_t(a.tiles_h));
    return p.dtype == CNHWC_BF16 ? launch_tilep_t<BF16>(a, int(blocks), st)
                                 : launch_tilep_t<F16>(a, int(blocks), st);
}

// p in dgrad terms (dy: N x Ho x Wo x C in, dx: N x H x W x C out);
// flip: read the filter rotated by 180 degrees; tune 1 keeps 7x7 on the
// one-tile-per-block kernel
int launch_tiled(const Prob& p, int flip, int tune, const void* dy, const void* w, void* dx, hipStream_t st) {
    if (dw_tiled_persist_applies(p, tune)) return launch_tiled_persistent(p, flip, dy, w, dx, st);
    TileArgs a{};
    a.flip = flip;
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.Ho = int(p.ho); a.Wo = int(p.wo);
    a.pad_h = p.pad_h; a.pad_w = p.pad_w;
    const int th = tile_th(int(p.r));
    a.tiles_h = int((p.h + th - 1) / th);
    a.tiles_w = int((p.w + kTileTW - 1) / kTileTW);
    a.cblocks = int((p.c + kTileCB - 1) / kTileCB);
    const int64_t blocks = int64_t(a.N) * a.tiles_h * a.tiles_w * a.cblocks;
    a.nblocks = int(blocks);
    a.remap = blocks % 8 == 0 ? 1 : 0;
    a.fd_tw = make_fastdiv(uint32_t(a.tiles_w));
    a.fd_th = make_fastdiv(uint32_t(a.tiles_h));
    a.fd_cb = make_fastdiv(uint32_t(a.cblocks));
    return p.dtype == CNHWC_BF16 ? launch_tile_t<BF16>(p, a, int(blocks), st)
                                 : launch_tile_t<F16>(p, a, int(blocks), st);
}

template <typename T, int SPLIT, int TB>
int launch_rot_inst(const RotArgs& a, int64_t blocks, size_t lds, hipStream_t st) {
    auto kern = dw_rotated_kernel<T, SPLIT, TB>;
    // dynamic LDS above 64 KiB must be opted into per kernel
    static bool attr_set = false;   // per instance; idempotent if raced
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024) != hipSuccess)
            return CNHWC_HIP_ERROR;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(256 * SPLIT), lds, st, a);
    return CNHWC_OK;
}

// p in dgrad terms; rot: correlate with the filter rotated by 180 degrees at
// padding R-1-pad (dgrad), else with the filter as stored at padding R-1-pad
int launch_rotated(const Prob& p, const Plan& pl, int rot, const void* dy, const void* w, void* dx,
                   hipStream_t st) {
    // tap groups: kRotSplit (two waves per SIMD at one block per CU); tune 1
    // asks for one group, tune 2 for two groups with 8-column slices whatever
    // the filter width (both with 8-column slices)
    const bool split = pl.tune != 1;
    const int tb = pl.tune == 1 || pl.tune == 2 ? kRotTB : rot_tb(p);
    RotArgs a{};
    size_t lds;
    if (!rot_geometry(p, tb, &a, &lds)) return CNHWC_UNSUPPORTED;
    a.rot = rot;
    a.dy = dy; a.w = w; a.dx = dx;
    a.dy_bytes = uint32_t(p.n * p.ho * p.wo * p.k * 2);
    a.w_bytes = uint32_t(p.k * p.r * p.s * 2);
    a.dx_bytes = uint32_t(p.n * p.h * p.w * p.c * 2);
    a.N = int(p.n); a.H = int(p.h); a.W = int(p.w); a.C = int(p.c); a.Ho = int(p.ho); a.Wo = int(p.wo);
    a.R = int(p.r); a.S = int(p.s);
    a.ph2 = int(p.r) - 1 - p.pad_h;
    a.pw2 = int(p.s) - 1 - p.pad_w;
    a.tiles_h = int((p.h + a.OHB - 1) / a.OHB);
    a.tiles_w = int((p.w + a.OWB - 1) / a.OWB);
    a.cblocks = int(p.c / kRotCB);
    const int64_t blocks = int64_t(a.N) * a.tiles_h * a.tiles_w * a.cblocks;
    if (!split) lds = size_t(a.IHB / 2) * a.row_dw * 4 + 2 * size_t(a.rpairs) * a.tslices * tb * kRotCB * 4;
    const bool bf = p.dtype == CNHWC_BF16;
    if (!split)
        return bf ? launch_rot_inst<BF16, 1, kRotTB>(a, blocks, lds, st)
                  : launch_rot_inst<F16, 1, kRotTB>(a, blocks, lds, st);
    switch (tb) {
    case 1: return bf ? launch_rot_inst<BF16, kRotSplit, 1>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 1>(a, blocks, lds, st);
    case 2: return bf ? launch_rot_inst<BF16, kRotSplit, 2>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 2>(a, blocks, lds, st);
    case 3: return bf ? launch_rot_inst<BF16, kRotSplit, 3>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 3>(a, blocks, lds, st);
    case 4: return bf ? launch_rot_inst<BF16, kRotSplit, 4>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 4>(a, blocks, lds, st);
    case 5: return bf ? launch_rot_inst<BF16, kRotSplit, 5>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 5>(a, blocks, lds, st);
    case 6: return bf ? launch_rot_inst<BF16, kRotSplit, 6>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 6>(a, blocks, lds, st);
    case 7: return bf ? launch_rot_inst<BF16, kRotSplit, 7>(a, blocks, lds, st) : launch_rot_inst<F16, kRotSplit, 7>(a, blocks, lds, st);
    default: return bf ? launch_rot_inst<BF16, kRotSplit, kRotTB>(a, blocks, lds, st)
                       : launch_rot_inst<F16, kRotSplit, kRotTB>(a, blocks, lds, st);
    }
}

}  // namespace

int launch_dgrad_dw_tiled(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                          hipStream_t st) {
    return launch_tiled(p, 0, pl.tune, dy, w, dx, st);
}

int launch_dgrad_dw_rotated(const Prob& p, const Plan& pl, const void* dy, const void* w, void* dx,
                            hipStream_t st) {
    return launch_rotated(p, pl, 1, dy, w, dx, st);
}

int launch_fwd_dw_tiled(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                        hipStream_t st) {
    return launch_tiled(fwd_as_dgrad(p), 1, pl.tune, x, w, y, st);
}

bool dw_tiled_persist_taken(const Prob& p, const Plan& pl) {
    if (pl.variant == CNHWC_VAR_DGRAD_DW_TILED) return dw_tiled_persist_applies(p, pl.tune);
    if (pl.variant == CNHWC_VAR_FWD_DW_TILED) return dw_tiled_persist_applies(fwd_as_dgrad(p), pl.tune);
    return false;
}

int launch_fwd_dw_rotated(const Prob& p, const Plan& pl, const void* x, const void* w, void* y,
                          hipStream_t st) {
    return launch_rotated(fwd_as_dgrad(p), pl, 0, x, w, y, st);
}

std::string fwd_dw_tiled_reason(const Prob& p) {
    if (p.stride != 1) return "the LDS-tiled depthwise forward needs stride 1";
    return dw_tiled_reason(fwd_as_dgrad(p));
}

std::string fwd_dw_rotated_reason(const Prob& p) {
    if (p.stride != 1) return "the rotated-filter depthwise forward needs stride 1";
    return dw_rotated_reason(fwd_as_dgrad(p));
}

}  // namespace cnhwc
