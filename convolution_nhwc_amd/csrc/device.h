// Device helpers for the gfx950 (CDNA4, wave64) kernels: 16-bit element types,
// raw buffer loads whose out-of-range lanes return zero, MFMA wrappers and
// round-to-nearest-even output conversion.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

#include "fastdiv.h"

namespace cnhwc {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Element tags.  Storage is always 16 bits; the tag picks the MFMA/dot
// instruction and the output conversion.
struct F16 {
    static constexpr bool is_bf16 = false;
};
struct BF16 {
    static constexpr bool is_bf16 = true;
};

// gfx9 buffer resource word 3 (raw buffer, no format conversion).
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// A byte offset at or above every view's num_records (views are < 2^31 bytes):
// loads from it return 0 and stores to it are dropped.
constexpr uint32_t kOob = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

__device__ inline i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ inline i32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ inline int buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ inline unsigned short buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
// Stores carry the non-temporal (streaming) cache policy: every kernel writes
// its outputs once and never reads them back, and streaming lines do not
// linger dirty in the XCD's L2 for the write-back at the end of the kernel.
constexpr int kStoreNT = 2;
__device__ inline void buf_store16(i32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStoreNT);
}
__device__ inline void buf_store8(i32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStoreNT);
}
__device__ inline void buf_store4(int v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStoreNT);
}
__device__ inline void buf_store2(unsigned short v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kStoreNT);
}

// D += A(16x32) * B(32x16) on the matrix cores.  Lane l supplies row l%16 of A
// and column l%16 of B, each with the eight reduction elements of slot group
// l/16; the result holds rows 4*(l/16)..+3 of column l%16.
template <typename T>
__device__ inline f32x4 mfma16x16x32(i32x4 a, i32x4 b, f32x4 c);
template <>
__device__ inline f32x4 mfma16x16x32<F16>(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x4 mfma16x16x32<BF16>(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2_f32_{f16,bf16}).
template <typename T>
__device__ inline float dot2(uint32_t a, uint32_t b, float acc);
template <>
__device__ inline float dot2<F16>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
}
template <>
__device__ inline float dot2<BF16>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// fp32 -> 16-bit storage, round to nearest even (v_cvt_pk_{f16,bf16}_f32).
template <typename T>
__device__ inline uint32_t pack2(float lo, float hi);
template <>
__device__ inline uint32_t pack2<F16>(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ inline uint32_t pack2<BF16>(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
template <typename T>
__device__ inline unsigned short pack1(float v) {
    return (unsigned short)(pack2<T>(v, 0.0f) & 0xffffu);
}

// 16-bit storage -> fp32.
template <typename T>
__device__ inline float to_f32(unsigned short b);
template <>
__device__ inline float to_f32<F16>(unsigned short b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
template <>
__device__ inline float to_f32<BF16>(unsigned short b) {
    return __builtin_bit_cast(float, uint32_t(b) << 16);
}

// Pair (lo half of a, lo half of b) / (hi half of a, hi half of b).
__device__ inline uint32_t pair_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ inline uint32_t pair_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---- asynchronous loads into LDS, waits, compile-time loops ----------------

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous 16-byte global -> LDS load: lane l writes lds_base + 16*l
// (lds_base must be wave-uniform: it goes to M0).
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

// LDS byte address (what ds_* instructions take) of a pointer into __shared__.
__device__ inline uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

template <int I>
using IC = std::integral_constant<int, I>;

// Compile-time loop: f(IC<0>{}), ..., f(IC<N-1>{}).
template <typename F, int... I>
__device__ inline void sfor_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(IC<I>{}), ...);
}
template <int N, typename F>
__device__ inline void sfor(F&& f) {
    sfor_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace cnhwc
