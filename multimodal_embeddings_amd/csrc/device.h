// device.h -- small device helpers shared by the gfx950 kernels of libube (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ube {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
    __bf16 b = (__bf16)v;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// Sums HP per-lane values over the 64 lanes of a wave at once: each exchange
// step halves the values a lane keeps (lane bits 5, 4, ... pick the half), the
// remaining steps finish the sums. Lane L then holds the total of value
// L / (64 / HP).
template <int HP>
__device__ __forceinline__ float lanes_reduce(const float (&p)[HP], int lane) {
    float cur[HP];
#pragma unroll
    for (int j = 0; j < HP; ++j) cur[j] = p[j];
    int m = 32;
#pragma unroll
    for (int n = HP; n > 1; n >>= 1, m >>= 1) {
        const bool up = lane & m;
#pragma unroll
        for (int j = 0; j < n / 2; ++j)
            cur[j] = (up ? cur[n / 2 + j] : cur[j]) + __shfl_xor(up ? cur[j] : cur[n / 2 + j], m, 64);
    }
    for (; m >= 1; m >>= 1) cur[0] += __shfl_xor(cur[0], m, 64);
    return cur[0];
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8). This remap gives every XCD one contiguous range of logical tiles, so
// tiles that share operands share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    int xcd = bid & 7, slot = bid >> 3;
    int q = nblocks >> 3, r = nblocks & 7;
    return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ void lds_dma16(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// One 4-byte DMA per lane: lane i's dword lands at lds_base + 4 i (lds_base uniform).
__device__ __forceinline__ void lds_dma4(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 4, 0, 0);
}

// Waits until at most N vector memory operations of this wave are outstanding (loads
// complete in issue order, so the oldest ones are then done).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence (the DMA of the next stage stays in
// flight); the empty asm keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Operand rows are 128 bytes (8 chunks of 16). gfx950's LDS has 64 banks (256
// bytes per cycle) and serves a 16-byte read for 16 lanes at a time: lanes
// reading rows r .. r+15 at the same logical chunk hit 16 distinct 16-byte bank
// groups when the chunk is XOR-ed with (row / 2) % 8 (row parity picks the
// 128-byte half of the 256-byte bank window).
__device__ __forceinline__ int swz(int row, int ch) { return ch ^ ((row >> 1) & 7); }

}  // namespace ube
