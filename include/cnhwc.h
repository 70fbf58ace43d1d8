/*
 * cnhwc.h -- C ABI of the gfx950 (MI355X) NHWC convolution library libcnhwc.so.
 *
 * Three passes of 2D convolution over fp16 or bf16 tensors with fp32
 * accumulation and one round-to-nearest-even rounding of each output element:
 *
 *   forward   y[n,ho,wo,k] = sum_{r,t,j} x[n, ho*s-pad_h+r, wo*s-pad_w+t, g*Cg+j] * w[k,r,t,j]
 *   dgrad     dx = the adjoint of that map (in x) applied to dy
 *   wgrad     dw[k,r,t,j] = sum_{n,ho,wo} dy[n,ho,wo,k] * x[n, ho*s-pad_h+r, wo*s-pad_w+t, g*Cg+j]
 *             (the adjoint of the map in w; the first page names it beside
 *             forward and dgrad as the pass that already had a 1x1 fast path)
 *
 * (cross-correlation, no filter flip; g = k / Kg, Cg = C/groups, Kg = K/groups;
 * x is zero outside the image).  The operations are those of three rocKE pull
 * requests: "perf(rocke/conv): add the pointwise fast path dgrad was missing"
 * (1x1 and general implicit-GEMM dgrad), "feat(rocke): split-C and grouped
 * LDS-halo direct conv fwd kernels" (direct forward, split-C with a reduce
 * pass, small groups merged block-diagonally, batch chunking past the 32-bit
 * buffer range) and "feat(rocke): channel-packed and large-filter depthwise
 * dgrad" (row-streaming and rotated-filter depthwise dgrad, per-axis padding).
 *
 * Layouts (all dense, row-major, 16-byte-aligned base pointers):
 *   x, dx  [N][H][W][C]          y, dy  [N][Ho][Wo][K]          w, dw  [K][R][S][C/groups]
 *   Ho = floor((H + 2*pad_h - R) / stride) + 1,  Wo = floor((W + 2*pad_w - S) / stride) + 1.
 *
 * Conventions shared by every entry point:
 *   - Pointers passed to cnhwc_fwd / cnhwc_dgrad / cnhwc_wgrad are DEVICE pointers on the
 *     current HIP device.  The caller allocates and owns every buffer,
 *     including the workspace; the library never allocates, frees or
 *     synchronises.  Inputs are read only; outputs are fully overwritten
 *     (positions no filter tap reaches are written as 0).
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the null stream).  A return of CNHWC_OK means the launches were
 *     enqueued, not that they finished.
 *   - A non-zero status leaves the outputs untouched, and cnhwc_last_error()
 *     returns a reason for it (thread-local, valid until the next call on the
 *     same thread).  The descriptor is checked in a fixed order and the first
 *     failing check is reported.
 *   - Inputs and outputs must not overlap.  Calls on one stream are ordered;
 *     calls on different streams that share an output race.
 */
#ifndef CNHWC_H
#define CNHWC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define CNHWC_OK 0
#define CNHWC_INVALID_ARG 1          /* descriptor or pointer argument invalid */
#define CNHWC_UNSUPPORTED 2          /* valid problem no kernel accepts (reason says why) */
#define CNHWC_WORKSPACE_TOO_SMALL 3  /* ws_bytes below cnhwc_workspace_size() */
#define CNHWC_MISALIGNED 4           /* a device pointer is not 16-byte aligned */
#define CNHWC_HIP_ERROR 5            /* the HIP runtime rejected a launch */

/* ---- element types and passes ------------------------------------------- */
#define CNHWC_F16 0
#define CNHWC_BF16 1

/* Pass numbers follow MIOpen's -F direction codes the first page's driver
 * parses: 1 = forward, 2 = backward data, 4 = backward weights. */
#define CNHWC_OP_FWD 1
#define CNHWC_OP_DGRAD 2
#define CNHWC_OP_WGRAD 4

/* Problem descriptor: the fields rocKE's DirectConvProblem carries (N, H, W,
 * C, K, filter rows R = KH, filter columns S = KW, stride, padding, groups),
 * with the column padding explicit rather than the "-1 means PAD" sentinel
 * ("feat(rocke): channel-packed and large-filter depthwise dgrad", Per-axis
 * padding).  One stride serves both axes; dilation is 1.
 * Valid: n,h,w,c,k,r,s >= 1; stride >= 1; pad_h, pad_w >= 0; groups >= 1 with
 * c % groups == 0 and k % groups == 0; Ho, Wo >= 1; dtype F16 or BF16;
 * reserved == 0. */
typedef struct cnhwc_problem {
    int64_t n, h, w, c, k, r, s;
    int32_t stride, pad_h, pad_w, groups;
    int32_t dtype;
    int32_t reserved;
} cnhwc_problem;

/* Kernel variants the dispatcher chooses among (cnhwc_plan names them). */
#define CNHWC_VAR_AUTO 0
#define CNHWC_VAR_DGRAD_POINTWISE 1  /* 1x1, stride 1, unpadded (grouped too): dX = dY * W per group on MFMA */
#define CNHWC_VAR_DGRAD_IGEMM 2      /* general R x S strided implicit-GEMM dgrad on MFMA */
#define CNHWC_VAR_DGRAD_DW_STREAM 3  /* depthwise dgrad, row-streaming, cpl channels per lane */
#define CNHWC_VAR_DGRAD_DW_ROTATED 4 /* depthwise dgrad, stride 1, rotated-filter tiled */
#define CNHWC_VAR_FWD_DIRECT 5       /* direct LDS-halo forward on MFMA, one pass */
#define CNHWC_VAR_FWD_SPLITC 6       /* direct forward, channel loop split; fp32 workspace + reduce pass */
#define CNHWC_VAR_FWD_GROUPED 7      /* grouped forward, small groups merged block-diagonally */
#define CNHWC_VAR_FWD_GENERIC 8      /* plain one-output-per-lane forward (any valid problem) */
#define CNHWC_VAR_DGRAD_GENERIC 9    /* plain one-output-per-lane dgrad (any valid problem) */
#define CNHWC_VAR_DGRAD_DW_TILED 10  /* depthwise dgrad, stride 1, 3x3/5x5/7x7, dY window tiled in LDS */
#define CNHWC_VAR_FWD_DW_TILED 11    /* depthwise forward, stride 1, 3x3/5x5/7x7: the tiled dgrad kernel
                                        on x with the filter rotated by 180 degrees, padding R-1-pad */
#define CNHWC_VAR_FWD_DW_ROTATED 12  /* depthwise forward, stride 1, filters up to 64 a side, any
                                        padding: the rotated-filter kernel with the filter as stored */
#define CNHWC_VAR_DGRAD_GROUPED 13   /* grouped dgrad, stride 1, small groups merged block-diagonally:
                                        the whole-row grouped kernel on dY with the filter rotated and
                                        transposed per group, padding R-1-pad */
#define CNHWC_VAR_WGRAD_GENERIC 14   /* plain one-weight-per-lane wgrad (any valid problem) */
#define CNHWC_VAR_WGRAD_POINTWISE 15 /* 1x1, stride 1, unpadded: split-K dW = dY^T X on MFMA, fp32
                                      * partials + reduce pass; the general kernel without the
                                      * per-row pixel gather, bit-identical to it */
#define CNHWC_VAR_WGRAD_SPLITK 16    /* general R x S strided wgrad: per tap, split-K implicit GEMM
                                      * on MFMA over the output pixels, fp32 partials + reduce pass */
#define CNHWC_VAR_DGRAD_SPLITK 17    /* split-K implicit-GEMM dgrad for few output tiles over a deep
                                      * reduction (small maps, many dY channels): the reduction steps
                                      * (filter taps x 64-deep dY channel chunks) of each tile split
                                      * over blocks, fp32 partials + the split reduce pass */
#define CNHWC_VAR_FWD_IGEMM 18       /* forward, stride 1, groups 1, pad <= filter - 1: the dgrad of the
                                      * 180-degree-rotated, transposed filter at padding R-1-pad on the
                                      * implicit-GEMM dgrad kernels (large maps); the transformed filter
                                      * goes to the workspace */

/* Output dims by the floor formula above, the column count following pad_w
 * ("feat(rocke): channel-packed and large-filter depthwise dgrad", Per-axis
 * padding, and its review's count of output columns when pad_w differs from
 * pad_h).  INVALID_ARG for a bad descriptor. */
int cnhwc_out_dims(const cnhwc_problem* prob, int64_t* ho, int64_t* wo);

/* Workspace bytes the chosen kernel of pass `op` needs.  The workspace is where
 * a split reduction keeps its fp32 partial sums until a second launch folds
 * them into the output ("feat(rocke): split-C and grouped LDS-halo direct conv
 * fwd kernels", description: the split_c variant and its second-pass
 * reduction); the same scheme serves split-K dgrad and wgrad.  Sizes: split_c * N * Ho * Wo
 * * K * 4 bytes of fp32 partial sums for the split-C forward, splits * N * H *
 * W * C * 4 bytes for the split-K dgrad (N: the largest batch chunk), K * R * S *
 * C * 2 bytes (the transformed filter) for the implicit-GEMM forward, splits * K * R
 * * S * C/groups * 4 bytes for the split-K wgrad kernels (splits: the pixel
 * splits of all batch chunks together), 0 for every other kernel.  Pass at
 * least this many bytes to cnhwc_fwd / cnhwc_dgrad / cnhwc_wgrad. */
int cnhwc_workspace_size(const cnhwc_problem* prob, int op, size_t* bytes);

/* The dispatcher's choice for pass `op`.  The pages' kernels ship with no
 * dispatcher ("feat(rocke): channel-packed and large-filter depthwise dgrad",
 * Motivation: the new binaries have no dispatcher wiring); this library adds
 * one, and this call exposes its decision.  Writes the kernel name (variant,
 * element type, tile or channels-per-lane) into name[0..cap) (truncated,
 * always NUL-terminated when cap > 0) and, if `variant` is not NULL, the
 * CNHWC_VAR_* number.  UNSUPPORTED with a reason when no kernel accepts. */
int cnhwc_plan(const cnhwc_problem* prob, int op, char* name, size_t cap, int32_t* variant);

/* Batch split of the launches for pass `op`: every per-image view of x/dx,
 * y/dy and the workspace must stay within the kernels' 32-bit buffer range
 * (2^31 - 1 bytes, or a lower limit set by the test override), so the batch runs as
 * balanced chunks of floor(N/chunks) or ceil(N/chunks) images ("feat(rocke):
 * split-C and grouped LDS-halo direct conv fwd kernels", supporting changes).
 * Writes up to `cap` chunk sizes (in images, in launch order) into counts and
 * their number into *nchunks.  UNSUPPORTED when one image alone is over the
 * limit. */
int cnhwc_chunk_plan(const cnhwc_problem* prob, int op, int64_t* counts, int64_t cap,
                     int64_t* nchunks);

/* Forward pass.  x: device [N,H,W,C]; w: device [K,R,S,C/groups];
 * y: device [N,Ho,Wo,K] (written); ws: device scratch of ws_bytes (may be NULL
 * when cnhwc_workspace_size() reports 0; its contents on return are
 * unspecified: split-C partial sums, or the implicit-GEMM forward's
 * transformed filter). */
int cnhwc_fwd(const cnhwc_problem* prob, const void* x, const void* w, void* y,
              void* ws, size_t ws_bytes, void* hip_stream);

/* Backward-data pass.  dy: device [N,Ho,Wo,K]; w: device [K,R,S,C/groups];
 * dx: device [N,H,W,C] (written, every element).  ws as for cnhwc_fwd (the
 * split-K kernel keeps one fp32 partial dx per reduction split there, summed
 * in ascending split order by a second launch). */
int cnhwc_dgrad(const cnhwc_problem* prob, const void* dy, const void* w, void* dx,
                void* ws, size_t ws_bytes, void* hip_stream);

/* Weight-gradient pass.  x: device [N,H,W,C]; dy: device [N,Ho,Wo,K];
 * dw: device [K,R,S,C/groups] (written, every element).  ws as for cnhwc_fwd
 * (the split-K kernels keep one fp32 partial dw per pixel split there; a
 * second launch sums the splits in a fixed order -- ascending within
 * contiguous split ranges, then the range sums ascending -- and rounds once;
 * each batch chunk contributes splits of its own). */
int cnhwc_wgrad(const cnhwc_problem* prob, const void* x, const void* dy, void* dw,
                void* ws, size_t ws_bytes, void* hip_stream);

/* Forward pass for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same dispatcher, kernels and results as cnhwc_fwd, with the workspace taken
 * from a static device array of CNHWC_STATIC_WS_BYTES that the library's code
 * object reserves on each GPU it runs on and keeps until the process ends.
 * The caller still passes x, w and y as for cnhwc_fwd.  Problems whose
 * workspace (cnhwc_workspace_size) exceeds CNHWC_STATIC_WS_BYTES are refused
 * with CNHWC_WORKSPACE_TOO_SMALL before any device call.  The call itself
 * allocates nothing (no hipMalloc / hipFree); its first call on a device looks
 * up the array's address there.  Every call on one GPU shares that GPU's
 * array and leaves its contents behind (nothing in it has to start at zero),
 * so calls that may overlap on one GPU -- on different streams, or from
 * different threads -- race on the workspace and must be ordered by the
 * caller. */
#define CNHWC_STATIC_WS_BYTES ((size_t)32 << 20)
int cnhwc_fwd_static_ws(const cnhwc_problem* prob, const void* x, const void* w, void* y,
                        void* hip_stream);

/* Reason for the last non-zero status on this thread ("" after success).  The
 * checks run in a fixed order and the first failing one is reported, as the
 * pages' C++ engine keeps its validators in the same order and with the same
 * reason text as the Python one ("feat(rocke): channel-packed and large-filter
 * depthwise dgrad", Technical Details, C++ engine).  The string is owned by
 * the library and valid until the next call on the same thread. */
const char* cnhwc_last_error(void);

/* Test-only override of the dispatcher's choices, thread-local.  It is an A/B
 * switch for tests and tuning sweeps, not a user knob: the kernel a shape
 * gets in normal use is the dispatcher's selection alone, and an override
 * only makes a comparison against that selection possible ("perf(rocke/conv):
 * add the pointwise fast path dgrad was missing", the commit that takes the
 * LDS-layout switch out of the sweep driver again because a sweep must only
 * measure kernels that dispatch can select).  A zero field
 * keeps the automatic choice.  variant: a CNHWC_VAR_* to force (the call fails
 * with UNSUPPORTED and the variant's reason if it cannot run the problem);
 * cpl: depthwise channels per lane (1, 2, 4 or 8); split_c: number of channel
 * splits for CNHWC_VAR_FWD_SPLITC or of reduction splits for
 * CNHWC_VAR_DGRAD_SPLITK (with the automatic variant it forces that split);
 * tune: a launch-shape knob of the chosen kernel (implicit-GEMM dgrad: 1 runs
 * every phase class on the ring kernel, 2 runs classes with two or more taps on
 * the dY-window kernel, 5 runs the persistent 8-wave kernel (taken by default
 * at stride >= 2 when C/groups is a multiple of 256 and K/groups of 128), a
 * value of 16 or more sets the ring kernel's pixels per tile, and for split-K any nonzero value keeps the ring kernel where the
 * filter-streaming one applies; direct forward: 1 forces the register-staged
 * kernel, 2 or 3 the input-window kernel (3 also where split-C over a small
 * map would take the filter-streaming kernel); implicit-GEMM forward: 1 keeps
 * the filter transform and the dgrad kernels for 1x1 shapes the pointwise row
 * kernel takes; split-K wgrad: the number of pixel splits per batch
 * chunk; depthwise rotated-filter: 1 runs one tap group, 2 two groups, both
 * with 8-column filter slices even for filters narrower than 8 columns;
 * depthwise LDS-tiled (dgrad and forward): 1 keeps 7x7 filters on the
 * one-tile-per-block kernel instead of the persistent one; other kernels
 * ignore it);
 * chunk_limit_bytes: the per-view byte limit of the chunk planner.  Pass NULL
 * to clear. */
typedef struct cnhwc_override {
    int32_t variant;
    int32_t cpl;
    int32_t split_c;
    int32_t tune;           /* kernel-specific launch-shape knob for tuning sweeps (0 = automatic) */
    int64_t chunk_limit_bytes;
} cnhwc_override;

int cnhwc_set_override(const cnhwc_override* ov);

#ifdef __cplusplus
}
#endif
#endif /* CNHWC_H */
