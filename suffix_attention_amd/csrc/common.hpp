// Device-side building blocks shared by the replay-attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace ls {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of a bfloat16 in memory

#define LS_LDS __attribute__((address_space(3)))


// ----------------------------------------------------------------------------------------
// Scalar conversions.  bf16 -> f32 is exact; f32 -> bf16 rounds to nearest-even in hardware.
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void store_f32(T* p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Pack two f32 to two bf16 (round to nearest-even) in one 32-bit word, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v{lo, hi}), bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of x held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0]: lanes 32..63 received lanes 0..31; r[1]: lanes 0..31 received lanes 32..63.
    return __uint_as_float((__lane_id() < 32) ? r[1] : r[0]);
}

// ----------------------------------------------------------------------------------------
// XCD-aware block order.  Workgroups are dispatched round-robin over the 8 XCDs of an
// MI355X, so hardware block b lands on XCD b % 8.  Renumbering as below gives each XCD a
// contiguous range of logical blocks, so blocks that share operands (the query tiles of
// one key range) run together behind one L2.  `n` must be a multiple of 8; callers pad
// the grid and let logical ids >= the real count return at once.
// ----------------------------------------------------------------------------------------
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical_block(int b, int n) {
    return (b % kXcds) * (n / kXcds) + b / kXcds;
}
inline int pad_grid(int n) { return (n + kXcds - 1) / kXcds * kXcds; }

// ----------------------------------------------------------------------------------------
// Direct global -> LDS copy of 16 bytes per lane, through a buffer resource over
// [base, base + bytes): lane l reads base + off and its bytes land at lds_wave_base + 16 * l
// (base, bytes and lds_wave_base uniform across the wave; lds_wave_base is an LDS byte
// address, see lds_addr).  Offsets past `bytes` read as 0.
//
// Issued as inline assembly, so the compiler's wait-count pass does not see it: the caller
// waits for the copies itself (wait_vm_all() before the barrier that publishes a tile).  Seen
// by the compiler, an LDS-writing load makes it guard LDS reads with waits it cannot always
// prove unnecessary (lgkmcnt(0) for the global form; vmcnt(0) in straight-line code for the
// buffer form), which drains the operand prefetch of the matrix loops.  The buffer form counts
// only in vmcnt.  The leading s_nop covers the M0 write just before it.
// ----------------------------------------------------------------------------------------
constexpr int kRawBufferWord3 = 0x00020000;  // 32-bit data format, no swizzle, no index
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b),
                 __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(b >> 32) & 0xffff),  // stride 0
                 __builtin_amdgcn_readfirstlane((int32_t)bytes), kRawBufferWord3};
}
// The same copy through a buffer resource built once (buffer_rsrc) for several copies.
__device__ __forceinline__ void dma16r(const i32x4& rsrc, uint32_t off, uint32_t lds_wave_base) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)));
}
__device__ __forceinline__ void dma16(const void* base, uint32_t bytes, uint32_t off, uint32_t lds_wave_base) {
    dma16r(buffer_rsrc(base, bytes), off, lds_wave_base);
}

// LDS byte address of a __shared__ object (folds to a constant for the kernel's own arrays).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const LS_LDS void*)p; }

// Reads at an LDS byte address.  The matrix loops form operand addresses as (lane base +
// buffer base) ^ step constant + row immediate: with buffers aligned to 1 KiB and the xor
// confined to bits 4..8, adding the buffer base first commutes with the xor, so each read costs
// one xor (the row offset goes into the instruction's immediate).
__device__ __forceinline__ bf16x8 lds_b128(uint32_t a) { return *(const LS_LDS bf16x8*)(uintptr_t)a; }
__device__ __forceinline__ f32x4 lds_f32x4(uint32_t a) { return *(const LS_LDS f32x4*)(uintptr_t)a; }

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 4 bf16 from LDS through the gfx950 transpose read.  Within each 16-lane group, lane i
// supplies the address of 4 consecutive elements; it receives element i % 4 of the chunks
// addressed by lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4 (a 4 x 16 block read as its
// transpose).
__device__ __forceinline__ i16x4 lds_read_tr4(const LS_LDS void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LS_LDS i16x4*)(p));
}
__device__ __forceinline__ i16x4 lds_tr4(uint32_t a) { return lds_read_tr4((const LS_LDS void*)(uintptr_t)a); }

// Matrix-core multiply-add with the accumulator held in AGPRs, for kernels built with
// VGPR-form matrix instructions (whose other accumulators feed vector-ALU work):
//   acc[32 x 32] += A[32 x 16] . B[16 x 32]   (v_mfma_f32_32x32x16_bf16)
// The compiler does not see this as a matrix instruction, so it does not model its hazards:
// the two wait states ahead of it cover a vector-ALU write of A or B just before it; a chain
// of these on one accumulator needs none (same-size back-to-back accumulation); the caller
// runs mfma_drain() before anything reads the accumulator, and keeps the accumulator out of
// vector-ALU code so that the compiler never moves it between these instructions.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Two independent ones back to back, with no wait states ahead of them: a single wave per SIMD
// issues roughly one instruction per four cycles, so every instruction saved counts.  The
// callers' A and B operands are LDS reads (covered by s_waitcnt) or vector-ALU results formed a
// whole step earlier; tests/test_mfma_hazards.py scans the built assembly and fails if a
// vector-ALU write of an operand ever lands within the two instructions ahead of one of them.
__device__ __forceinline__ void mfma32_agpr2(f32x16& acc0, const bf16x8& a0, const bf16x8& b0, f32x16& acc1,
                                             const bf16x8& a1, const bf16x8& b1) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %4, %5, %1"
                 : "+a"(acc0), "+a"(acc1)
                 : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}

// Enough wait states for any matrix instruction in flight to retire before its result is read
// by inline assembly, which the compiler's hazard tracking does not see (the longest,
// 32x32x16, needs fewer than 20).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// x * f for an accumulator element held in an AGPR, computed in place (through one scratch VGPR), so
// that the accumulator never has to leave the AGPRs.  Call mfma_drain() before the first one
// if a matrix instruction may still be writing x, and agpr_write_gap() before the next matrix
// instruction reads it.
__device__ __forceinline__ float agpr_scaled(float x, float f) {
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(f));
    return x;
}

// Wait states between a v_accvgpr_write made in inline assembly (which the compiler's hazard
// tracking does not see) and a matrix instruction reading that accumulator.
__device__ __forceinline__ void agpr_write_gap() { asm volatile("s_nop 7" ::: "memory"); }

}  // namespace ls
