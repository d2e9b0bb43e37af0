// Device helpers shared by the forward and backward attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format; no
// swizzle, no stride): loads through it are range-checked against the
// resource's byte count and return 0 past it.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Max / sum with the lane 32 apart (v_permlane32_swap: both halves see both values).
__device__ __forceinline__ float max_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row of the 32x32 MFMA accumulator held in register v of a lane in half h.
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// LDS column of key `kk` (0..63) inside a V^T row.  Keys are permuted within
// each group of 16 so that the eight keys one lane contracts over in a P*V
// MFMA are adjacent (one 16-byte read); see the P fragment layout below.
__device__ __forceinline__ int vt_slot(int kk) {
    const int c = kk >> 4, a = (kk >> 3) & 1, hh = (kk >> 2) & 1, b = kk & 3;
    return 16 * c + 8 * hh + 4 * a + b;
}

// Scheduling pattern for N MFMAs whose operands come from R LDS reads each:
// issue the reads of the first AHEAD MFMAs, then alternate one MFMA with the
// reads of a further one, so each MFMA's operand was requested about AHEAD
// MFMAs (~32 cycles each) earlier.
constexpr int kLdsAhead = 6;
template <int N, int AHEAD, int R = 1>
__device__ __forceinline__ void pipeline_lds_mfma() {
    constexpr int A = AHEAD < N ? AHEAD : N;
    __builtin_amdgcn_sched_group_barrier(0x100, A * R, 0);      // DS reads
#pragma unroll
    for (int i = 0; i < N - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);      // DS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lanes 4r .. 4r+3 each name 8 bytes (four 16-bit values) that together
// form row r of a 4 x 16 matrix; lane i of the group receives column i, i.e.
// value i of rows 0, 1, 2, 3.  (Measured on the device with an in-bounds probe.)
__device__ __forceinline__ i16x4 ds_read_tr16(const lds_u8* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<lds_u8*>(p)));
}

// Barrier that orders LDS traffic only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One LDS-DMA instruction: each lane's 16 bytes at global offset voff of the
// buffer rsrc land at LDS byte lds + 16 * lane.  Issued through inline
// assembly so that the compiler does not order every LDS read behind every
// outstanding copy; the kernel waits for its own copies (vmcnt) before the
// barrier that publishes a tile.  M0 is a reserved register for the compiler:
// naming it in the clobber list is not honoured (clang warns that reserved
// registers may not be preserved), so correctness rests on nothing else in
// these kernels using M0, which the ISA test checks on every build.
// The LDS address is wave-uniform by construction (stage, block and wave
// index); readfirstlane tells the compiler so.
__device__ __forceinline__ void lds_dma16(uint32_t lds, u32x4 rsrc, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 : : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory");
}
// The same copy with compile-time offsets: LDS byte lds + LDS_OFF, source
// offset voff + SRC_OFF (SRC_OFF through the instruction's scalar offset).
// Only the base addresses occupy registers, so a loop over many blocks keeps
// nothing per block live.
template <int LDS_OFF, int SRC_OFF>
__device__ __forceinline__ void lds_dma16_at(uint32_t lds, u32x4 rsrc, uint32_t voff) {
    if constexpr (SRC_OFF == 0) {
        asm volatile("s_add_u32 m0, %0, %3\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     : : "s"(lds), "v"(voff), "s"(rsrc), "i"(LDS_OFF) : "memory", "scc");
    } else {
        uint32_t so;
        asm volatile("s_add_u32 m0, %1, %4\n\ts_mov_b32 %0, %5\n\tbuffer_load_dwordx4 %2, %3, %0 offen lds"
                     : "=&s"(so) : "s"(lds), "v"(voff), "s"(rsrc), "i"(LDS_OFF), "i"(SRC_OFF) : "memory", "scc");
    }
}
__device__ __forceinline__ void wait_lds_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Race-check build (compile with -DFA_POISON_STAGES=1): before a wave issues a
// copy into a ring stage, it fills the 1 KiB LDS block the copy will land in
// with NaN.  The poison goes in after the barrier that ends the last read of
// the stage's previous tile; a read of the stage that lagged behind that
// barrier, or ran ahead of the copy's wait, would see NaN instead of data, so
// this build's outputs equal the normal build's bit for bit only if no such
// race exists.
#ifndef FA_POISON_STAGES
#define FA_POISON_STAGES 0
#endif
__device__ __forceinline__ void poison_block(uint32_t lds) {
    if constexpr (FA_POISON_STAGES != 0) {
        const uint32_t addr = lds + 16u * (threadIdx.x & 63u);
        const u32x4 nan = {0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u};
        asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(nan) : "memory");
    }
}

// f(std::integral_constant<int, I>) for I = B .. E-1, each a compile-time constant.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Buffer resource words for a byte range [base, base + bytes) (the layout
// __builtin_amdgcn_make_buffer_rsrc builds), for the inline-assembly copies.
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, bytes,
                 static_cast<uint32_t>(kBufferFlags)};
}

// LDS byte address of a __shared__ object (what M0 takes).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const uint8_t*)p));
}

// Per-lane global offset of 1 KiB LDS block b of a region of `rows` padded
// rows: row r of the region holds `data` 16-byte granules of global row r
// (global row stride `stride` bytes) followed by one pad granule.  A lane on a
// pad granule or past the last row gets an offset past any buffer (it reads
// zero and moves no data).
__device__ __forceinline__ uint32_t dma_lane_offset(int b, int lane, int data, uint32_t stride, int rows) {
    const int g = 64 * b + lane, row = g / (data + 1), col = g - (data + 1) * row;
    return col < data && row < rows ? static_cast<uint32_t>(row) * stride + 16 * col : 0x40000000u;
}

// Bytes of LDS a region of padded rows occupies: whole 1 KiB copy blocks.
constexpr int dma_region_bytes(int bytes) { return (bytes + 1023) / 1024 * 1024; }
}  // namespace
}  // namespace fa
