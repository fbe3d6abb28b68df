// Device helpers shared by the forward and backward kernels: vector types,
// the bf16 MFMA step, the XOR swizzle of [token][d] tiles in LDS, the packed
// token-table word and window-local coordinates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_geometry.h"

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8; // MI355X: workgroups are dealt to 8 XCDs round-robin

// Blocks are dealt to the XCDs round-robin (block i to XCD i % 8).  This maps
// a block id to a work index so that each XCD walks a contiguous range of
// work items: the heads of one window run side by side on one XCD and read
// whole token rows together, and neighbouring windows share that XCD's L2.
__device__ inline int64_t xcd_work_index(int64_t bid, int64_t total) {
    int64_t q = total / kXcds, r = total % kXcds;
    int64_t x = bid % kXcds, k = bid / kXcds;
    return x * q + (x < r ? x : r) + k;
}

constexpr int kLdsBytes = 160 * 1024; // gfx950 LDS per compute unit
#ifndef SWA_MFMA_K32
#define SWA_MFMA_K32 1
#endif
// 1: 32-deep v_mfma_f32_16x16x32_bf16; 0: pairs of 16-deep v_mfma_f32_16x16x16_bf16
// fed from the same 16-byte fragments (low and high 8 bytes as two k-steps).
// Both take 16 cycles on gfx950, so the 32-deep form has twice the throughput.
// Every accumulator chain uses a single opcode: back-to-back dependent MFMAs of
// different opcodes on one accumulator gave wrong sums on gfx950 with this
// compiler's schedules, same-opcode chains do not.
constexpr bool kMfmaK32 = SWA_MFMA_K32 != 0;

__device__ inline i16x4 half_lo(bf16x8 x) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    return __builtin_bit_cast(i16x4, u32x2{u[0], u[1]});
}
__device__ inline i16x4 half_hi(bf16x8 x) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    return __builtin_bit_cast(i16x4, u32x2{u[2], u[3]});
}
// acc += A B over a 32-deep step, A and B as 16-byte lane fragments
__device__ inline f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 acc) {
    if (kMfmaK32) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(half_lo(a), half_lo(b), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(half_hi(a), half_hi(b), acc, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kRowMask = (1 << 28) - 1; // packed table word: source row + 1 in bits 0..27

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }


typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline unsigned pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 16-byte chunk slot of logical chunk c in K row m (rows of D bf16): an XOR
// with a key that changes every 128 bytes of rows, so that 16 consecutive rows
// read at one logical chunk spread over the banks
template <int D>
__device__ inline int k_slot(int m, int c) {
    constexpr int CH = D / 8;
    constexpr int ROWS_PER_128B = D * 2 >= 128 ? 1 : 128 / (D * 2);
    return c ^ ((m / ROWS_PER_128B) % CH);
}

// Logical chunk that a 1 KB copy lane lands in its slot of row m (the swizzle
// is an XOR, so self-inverse).  Each copy moves 64 / (D / 8) rows; when that
// is a multiple of the swizzle period (D <= 64) the row within the copy is
// enough, otherwise the key comes from the row itself.
template <int D>
__device__ inline int copy_chunk(int m, int lane) {
    constexpr int CH = D / 8;
    constexpr int RPC = 64 / CH;
    constexpr int ROWS_PER_128B = D * 2 >= 128 ? 1 : 128 / (D * 2);
    constexpr int PERIOD = ROWS_PER_128B * CH;
    return k_slot<D>(RPC % PERIOD == 0 ? lane / CH : m, lane % CH);
}

// window-local coordinates of local index n
__device__ inline void local_coords(const Geometry& g, int n, int& lt, int& ly, int& lx) {
    const uint32_t r = fdiv(g.fd_win2, (uint32_t)n);
    lx = n - (int)r * g.win[2];
    lt = (int)fdiv(g.fd_win1, r);
    ly = (int)r - lt * g.win[1];
}

// Per-window token tables in LDS, used by the fp32 kernels:
//   kword[m], qword[n]  mask words (see swa_geometry.h)
//   rowi[n]             row index of token n in the tensors read and written:
//                       the real token index (fused) or window*N + n (staged);
//                       -1 for pad tokens and slots past N
__device__ inline void fill_token_tables(const Geometry& g, int64_t wi, bool staged, int NP,
                                         int* kword, int* qword, int* rowi) {
    int b, wc[3];
    window_coords(g, wi, b, wc);
    for (int n = threadIdx.x; n < NP; n += blockDim.x) {
        if (n < g.N) {
            TokenInfo ti = token_info(g, b, wc, n);
            kword[n] = key_word(ti);
            qword[n] = query_word(ti);
            rowi[n] = ti.tok < 0 ? -1 : (staged ? (int)(wi * g.N + n) : (int)ti.tok);
        } else {
            kword[n] = kNoKey;
            // largest qb, so that qb - kb stays inside the bias table for every key
            qword[n] = kPadQuery | (g.table_size - 1);
            rowi[n] = -1;
        }
    }
}

} // namespace swa
