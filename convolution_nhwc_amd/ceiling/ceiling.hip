// Machine-ceiling microbenchmarks for the benchmark's roofline report
// (libcnhwc_ceiling.so; not part of the convolution library's C ABI).
//
// Each kernel measures one limit the convolution kernels run into on MI355X,
// so a measured time can be reported against what the machine delivers under
// the same kind of load as well as against the vendor peak:
//   - HBM streams with R reads to 1 write (R = 1..4) and a read-only stream,
//     16-byte non-temporal accesses, grid-stride over buffers much larger than
//     the 256 MB Infinity Cache;
//   - dense MFMA 16x16x32 f16 issue with independent accumulators at a chosen
//     number of waves per SIMD;
//   - v_dot2_f32_f16 issue (two multiply-adds a lane per instruction) at a
//     chosen number of waves per SIMD;
//   - LDS read bandwidth with 16-byte reads at 1 to 4 blocks of 4 waves a CU;
//   - an empty kernel, launched back to back (dispatch and drain cost).
// Every kernel writes a result that depends on all its work, so nothing is
// optimised away; a result is stored only under a data-dependent condition
// that the inputs never meet, and always to element 0 of the sink buffer.
// The host times launches with events on the stream it passes in.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ inline i32x4 ld_nt(const i32x4* p) { return __builtin_nontemporal_load(p); }
__device__ inline void st_nt(i32x4 v, i32x4* p) { __builtin_nontemporal_store(v, p); }

// R sources of n 16-byte elements each; R = 0 reads src[0] only (read-only
// stream, nothing written but the sink); otherwise dst[i] = xor of the R
// sources' element i.
template <int R>
__global__ __launch_bounds__(kThreads) void stream_kernel(const i32x4* __restrict__ s0,
                                                          const i32x4* __restrict__ s1,
                                                          const i32x4* __restrict__ s2,
                                                          const i32x4* __restrict__ s3,
                                                          i32x4* __restrict__ dst, int64_t n,
                                                          int* __restrict__ sink) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    i32x4 acc = {0, 0, 0, 0};
    for (int64_t base = int64_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n;
         base += stride * kUnroll) {
        i32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + int64_t(u) * kThreads;
            v[u] = i < n ? ld_nt(s0 + i) : i32x4{0, 0, 0, 0};
            if constexpr (R >= 2) v[u] ^= i < n ? ld_nt(s1 + i) : i32x4{0, 0, 0, 0};
            if constexpr (R >= 3) v[u] ^= i < n ? ld_nt(s2 + i) : i32x4{0, 0, 0, 0};
            if constexpr (R >= 4) v[u] ^= i < n ? ld_nt(s3 + i) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + int64_t(u) * kThreads;
            if constexpr (R == 0) acc ^= v[u];
            else if (i < n) st_nt(v[u], dst + i);
        }
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5a5a1234) sink[0] = 1;
}

// 8 independent accumulator chains of MFMA 16x16x32 f16 per wave.  The
// instruction is written out so that each chain accumulates in place: left to
// the compiler, the loop-carried accumulators are rotated through extra
// register moves between the matrix instructions, which measures those moves
// rather than the matrix cores.  Seven other products separate each chain's
// consecutive instructions, far more than the dependency needs.
#define CNHWC_MFMA_CHAIN(c) asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %1, %0" : "+a"(c) : "v"(a))
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float* __restrict__ sink) {
    const _Float16 a0 = _Float16(float(threadIdx.x & 7) * 0.001f);
    const f16x8 a = {a0, a0, a0, a0, a0, a0, a0, a0};
    const float z = float(threadIdx.x) * 1e-7f;
    f32x4 c0 = {z, 0.f, 0.f, 0.f}, c1 = {z + 1.f, 0.f, 0.f, 0.f}, c2 = {z + 2.f, 0.f, 0.f, 0.f},
          c3 = {z + 3.f, 0.f, 0.f, 0.f}, c4 = {z + 4.f, 0.f, 0.f, 0.f}, c5 = {z + 5.f, 0.f, 0.f, 0.f},
          c6 = {z + 6.f, 0.f, 0.f, 0.f}, c7 = {z + 7.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
        CNHWC_MFMA_CHAIN(c0); CNHWC_MFMA_CHAIN(c1); CNHWC_MFMA_CHAIN(c2); CNHWC_MFMA_CHAIN(c3);
        CNHWC_MFMA_CHAIN(c4); CNHWC_MFMA_CHAIN(c5); CNHWC_MFMA_CHAIN(c6); CNHWC_MFMA_CHAIN(c7);
    }
    // let the last products retire before their accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const f32x4 s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    if (s[0] + s[1] + s[2] + s[3] == -1.0f) sink[0] = s[0];
}
#undef CNHWC_MFMA_CHAIN

// 8 independent v_dot2_f32_f16 chains per lane.
__global__ __launch_bounds__(kThreads) void dot2_kernel(int iters, float* __restrict__ sink) {
    const _Float16 a0 = _Float16(float(threadIdx.x & 7) * 0.001f);
    const f16x2 a = {a0, a0};
    const f16x2 b = {a0, a0};
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = float(j);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_fdot2(a, b, acc[j], false);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j];
    if (s == -1.0f) sink[0] = s;
}

// LDS read bandwidth: every lane reads 16 bytes per ds_read_b128 from a
// 64 KiB block-local buffer, walking it so consecutive reads of a wave cover
// distinct, conflict-free 1 KiB rows; 8 reads in flight per lane.
__global__ __launch_bounds__(kThreads) void lds_kernel(int iters, int* __restrict__ sink) {
    __shared__ i32x4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += kThreads) buf[i] = i32x4{i, i + 1, i + 2, i + 3};
    __syncthreads();
    i32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = i32x4{0, 0, 0, 0};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] ^= buf[(((i * 8 + j + wave * 16) & 63) << 6) + lane];
    }
    i32x4 s = acc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) s ^= acc[j];
    if ((s.x ^ s.y ^ s.z ^ s.w) == 0x7e57ab1e) sink[0] = 1;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// reads: 0 = read-only stream over s[0]; 1..4 = that many sources, one
// destination.  n16: 16-byte elements per buffer.  Returns a hipError_t.
int ceiling_stream(int reads, const void* s0, const void* s1, const void* s2, const void* s3, void* dst,
                   int64_t n16, int blocks, void* sink, void* stream) {
    const auto a = static_cast<const i32x4*>(s0);
    const auto b = static_cast<const i32x4*>(s1);
    const auto c = static_cast<const i32x4*>(s2);
    const auto d = static_cast<const i32x4*>(s3);
    auto o = static_cast<i32x4*>(dst);
    auto k = static_cast<int*>(sink);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (reads) {
    case 0: hipLaunchKernelGGL(stream_kernel<0>, dim3(blocks), dim3(kThreads), 0, st, a, b, c, d, o, n16, k); break;
    case 1: hipLaunchKernelGGL(stream_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, a, b, c, d, o, n16, k); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, dim3(blocks), dim3(kThreads), 0, st, a, b, c, d, o, n16, k); break;
    case 3: hipLaunchKernelGGL(stream_kernel<3>, dim3(blocks), dim3(kThreads), 0, st, a, b, c, d, o, n16, k); break;
    case 4: hipLaunchKernelGGL(stream_kernel<4>, dim3(blocks), dim3(kThreads), 0, st, a, b, c, d, o, n16, k); break;
    default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}

// One block of 4 waves (one a SIMD) per `blocks`; 8 MFMA 16x16x32 chains of
// `iters` each per wave: blocks * 4 * iters * 8 * 16384 flops.
int ceiling_mfma(int blocks, int iters, void* sink, void* stream) {
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<float*>(sink));
    return int(hipGetLastError());
}

// blocks * 256 lanes * iters * 8 dot2 instructions, 4 flops a lane each.
int ceiling_dot2(int blocks, int iters, void* sink, void* stream) {
    hipLaunchKernelGGL(dot2_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<float*>(sink));
    return int(hipGetLastError());
}

// blocks * 256 lanes * iters * 8 reads of 16 bytes from LDS.
int ceiling_lds(int blocks, int iters, void* sink, void* stream) {
    hipLaunchKernelGGL(lds_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<int*>(sink));
    return int(hipGetLastError());
}

int ceiling_empty(int blocks, void* stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream));
    return int(hipGetLastError());
}

}  // extern "C"
