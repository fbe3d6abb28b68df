// Device helpers of the streaming bf16 schedule, shared by the streaming
// attention kernel (swa_kernels.hip) and the fused projection-attention layer
// kernel (swa_layer.hip): the LDS layout, the barriers, the unit decoder, the
// loader-wave copies and the two halves of a query tile's arithmetic.
#pragma once

#include "swa_device.h"
#include "swa_geometry.h"

namespace swa {

// --------------------------------------------------------------------------
// bf16 attention, streaming schedule: persistent blocks with LDS double buffers.
//
// The same per-tile arithmetic as above, instruction for instruction (both
// schedules give bit-identical outputs), but a block stays resident and walks
// a sequence of (window, head) units.  Each XCD (block % 8) owns a contiguous
// range of units and its blocks interleave over it, so an XCD works on the
// heads of a few neighbouring windows at a time.
//
// A block has one wave per 16-query tile (windows of up to 9 tiles) plus
// NL loader waves.  Only the loaders read global memory: they build
// each unit's token table and copy its K, Q and V straight into LDS with
// global_load_lds (16 bytes per lane, eight lanes per 128-byte token row, so
// every request is a whole line), [token][d] with 16-byte chunks
// XOR-swizzled by row (the source chunk a lane fetches is chosen so that the
// copy lands swizzled).  Loader wave j owns a contiguous range of token rows:
// it writes their table words and issues their copies, so it never reads
// what the other loader wrote.
//
// Unit i takes two block barriers: A_i (its K and Q are in LDS) and B_i (its
// V is in LDS; its K and Q are no longer read).  K, Q and V have two buffers
// each, so a copy can start 1.5 units before its data is needed:
//   after A_i  the loaders issue V(i+1)          (its buffer held V(i-1));
//   after B_i  they issue K(i+2), Q(i+2)         (their buffers held K(i), Q(i)).
// Token tables are built three units ahead and the source offsets of each
// batch are read from its table while the batch before it is awaited, so the
// copies leave right after each barrier.
// Copies are issued in the order K0 Q0 V0 K1 Q1 | V(i+1) K(i+2) Q(i+2) ...,
// and a loader issues nothing else, so each wait is an exact vmcnt count
// (vector memory operations of a wave complete in order): before A_i at most
// V(i) and K/Q(i+1) may be outstanding, before B_i at most K/Q(i+1) and V(i+1).
//
// Compute waves: between A_i and B_i, S^T = K Q^T, bias, mask and softmax,
// leaving bf16 P in registers; between B_i and A_(i+1), O^T = V^T P^T, then
// the O tile goes to the wave's rows of an LDS staging buffer and leaves as
// whole 128-byte token rows through buffer stores (lanes of pad queries store
// out of range, which the buffer range check drops).  The two roles run
// separate loops with the same number of barriers, and the barriers fence LDS
// only: a full fence would wait for every store in flight.  The PV product
// reads V^T fragments with ds_read_b64_tr_b16, which hands lane i of each
// 16-lane group element i of the 4 rows its group addresses.
// --------------------------------------------------------------------------
constexpr float kLn2 = 0.6931471805599453f; // natural log of 2: log-sum-exp from log2 units
constexpr int kBufs = 2;       // buffers each of K, Q and V
constexpr int kTableSlots = 4; // token tables of units i .. i+3
constexpr int kStreamMaxTiles = 9;
constexpr int kStreamMaxTiles128 = 5; // 128-wide heads: seven buffers of 5 tiles fill the LDS

struct StreamLds {
    int NP, TSP;   // padded keys; bias table entries per head slice (multiple of 64)
    bool bias_resident;
    size_t tb;     // bytes of one [NP][D] bf16 buffer
    size_t k0, q0, v0, o0, bias, kb4, slot0, slot_bytes, total;
};

__host__ __device__ inline StreamLds stream_lds_with(const Geometry& g, bool bias_resident) {
    StreamLds L;
    L.NP = (g.N + 15) / 16 * 16;
    L.TSP = (g.table_size + 63) / 64 * 64;
    L.bias_resident = bias_resident;
    L.tb = (size_t)L.NP * g.head_dim * 2;
    L.k0 = 0;
    L.q0 = L.k0 + kBufs * L.tb;
    L.v0 = L.q0 + kBufs * L.tb;
    L.o0 = L.v0 + kBufs * L.tb;
    L.bias = L.o0 + L.tb;
    L.kb4 = L.bias + (size_t)(bias_resident ? g.heads : kTableSlots) * L.TSP * 4;
    L.slot0 = L.kb4 + (size_t)L.NP * 4;
    L.slot_bytes = (size_t)L.NP * 4; // one packed word per token: (row + 1) | mask field << 28
    L.total = L.slot0 + kTableSlots * L.slot_bytes;
    return L;
}

// Every head's bias stays in LDS when that costs no resident block per CU.
__host__ __device__ inline StreamLds stream_lds(const Geometry& g) {
    const StreamLds S = stream_lds_with(g, false);
    const int tsp = (g.table_size + 63) / 64 * 64;
    if ((size_t)g.heads * tsp * 4 <= (size_t)24 * 1024) {
        const StreamLds R = stream_lds_with(g, true);
        if (R.total <= (size_t)kLdsBytes && kLdsBytes / R.total >= kLdsBytes / S.total) return R;
    }
    return S;
}

constexpr uint32_t kOutOfRange = 0x80000000u; // buffer offset past every tensor the schedule takes
constexpr int kBufferWord3 = 0x00020000;     // raw buffer resource, 32-bit data format
constexpr int kNonTemporal = 2;              // cache policy of read-once / write-once traffic (nt)

// Waits until at most min(n, 63) vector-memory operations of this wave are
// outstanding; n must be wave-uniform (a scalar branch picks the immediate).
__device__ inline void wait_vmcnt_le(int n) {
    switch (n < 63 ? n : 63) {
#define SWA_VM(c) \
    case c: __builtin_amdgcn_s_waitcnt(vmcnt_imm(c)); break;
#define SWA_VM8(c) SWA_VM(c) SWA_VM(c + 1) SWA_VM(c + 2) SWA_VM(c + 3) SWA_VM(c + 4) SWA_VM(c + 5) SWA_VM(c + 6) SWA_VM(c + 7)
        SWA_VM8(0) SWA_VM8(8) SWA_VM8(16) SWA_VM8(24) SWA_VM8(32) SWA_VM8(40) SWA_VM8(48) SWA_VM8(56)
#undef SWA_VM8
#undef SWA_VM
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

// Block barrier that orders LDS accesses only: waits for this wave's LDS
// operations, not for its global loads and stores.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same barrier for the loader waves, whose only LDS writes are table
// words (covered by the lgkmcnt wait) and copies they have already waited for
// with vmcnt.  A release fence here would make the compiler wait for every
// LDS copy in flight (vmcnt(0)), which drains the pipeline; the empty asm
// statements only keep the compiler from moving LDS accesses across it.
__device__ inline void loader_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// unit -> (window, head, batch item, window coordinates)
struct Unit {
    uint32_t wi;
    int h, b, wc[3];
};

__device__ inline Unit decode_unit(const Geometry& g, uint32_t u) {
    Unit U;
    U.wi = fdiv(g.fd_heads, u);
    U.h = (int)(u - U.wi * (uint32_t)g.heads);
    U.b = (int)fdiv(g.fd_nW, U.wi);
    const uint32_t r = U.wi - (uint32_t)U.b * (uint32_t)g.nW;
    const uint32_t r2 = fdiv(g.fd_nwin2, r);
    U.wc[2] = (int)(r - r2 * (uint32_t)g.nwin[2]);
    U.wc[0] = (int)fdiv(g.fd_nwin1, r2);
    U.wc[1] = (int)(r2 - (uint32_t)U.wc[0] * (uint32_t)g.nwin[1]);
    return U;
}

// The 1 KB copies (per tensor) of loader wave j: [c0, c1), covering token rows
// [c0 * RPC, c1 * RPC) with RPC = 64 / (D / 8) rows per copy.
struct LoaderRange {
    int c0, c1;
};

__host__ __device__ inline LoaderRange loader_range(const Geometry& g, const StreamLds& L, int j, int nl) {
    const int ncopy = L.NP * (g.head_dim / 8) / 64;
    return LoaderRange{ncopy * j / nl, ncopy * (j + 1) / nl};
}

// Copies loader wave j issues with a unit's K and Q (plus the streamed bias
// slice for loader 0), and with its V.
__host__ __device__ inline int loader_kq_copies(const Geometry& g, const StreamLds& L, int j, int nl) {
    const LoaderRange R = loader_range(g, L, j, nl);
    return 2 * (R.c1 - R.c0) + (j == 0 && !L.bias_resident ? L.TSP / 64 : 0);
}
__host__ __device__ inline int loader_v_copies(const Geometry& g, const StreamLds& L, int j, int nl) {
    const LoaderRange R = loader_range(g, L, j, nl);
    return R.c1 - R.c0;
}

// Table words of loader j's rows of unit uu, into slot s: (source row + 1, 0
// for pad) | mask field << 28, the mask field holding the wrapped flags with
// pad in bit 3 (15 past N).
template <int D>
__device__ inline void stream_table(const Geometry& g, const StreamLds& L, unsigned char* smem, LoaderRange R,
                                    int lane, uint32_t uu, int s, int staged) {
    constexpr int RPC = 64 / (D / 8);
    const int N = g.N;
    const Unit U = decode_unit(g, uu);
    int* tw = (int*)(smem + L.slot0 + s * L.slot_bytes);
    for (int n = R.c0 * RPC + lane; n < R.c1 * RPC; n += 64) {
        if (n < N) {
            int l[3];
            local_coords(g, n, l[0], l[1], l[2]);
            int region = 0, tok = U.b;
            bool is_pad = false;
#pragma unroll
            for (int a = 0; a < 3; a++) {
                const int cr = U.wc[a] * g.win[a] + l[a];
                int c = cr + g.shift[a];
                if (c >= g.pad[a]) c -= g.pad[a];
                is_pad |= c >= g.ext[a];
                if (!g.cyc[a] && cr >= g.pad[a] - g.shift[a]) region |= 1 << a;
                tok = tok * g.ext[a] + c;
            }
            const int row = is_pad ? -1 : (staged ? (int)(U.wi * (uint32_t)N + n) : tok);
            tw[n] = (row + 1) | ((region | (is_pad ? 8 : 0)) << 28);
        } else {
            tw[n] = 15 << 28;
        }
    }
    // the copies read table words other lanes of this wave just wrote
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Most 1 KB copies per tensor a loader wave issues for a unit.
template <int D, int KT_FIXED, int NL>
constexpr int loader_max_copies() {
    return ((KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles) * 16 * (D / 8) / 64 + NL - 1) / NL;
}

// Source element offsets (within a head's slice of a token row) of loader j's
// copies for the unit whose table is in slot s: 1 KB per copy, 8 lanes per
// 128-byte token row, the source chunk chosen so that the row lands swizzled.
// Pad rows copy row 0 (finite values that get weight exactly 0, or outputs
// that are never stored).  All table reads are issued before any is used.
template <int D, int MAXC, bool EXACT>
__device__ inline void stream_offsets(const Geometry& g, const StreamLds& L, const unsigned char* smem, LoaderRange R,
                                      int lane, int s, uint32_t (&off)[MAXC]) {
    constexpr int CH = D / 8;
    constexpr int RPC = 64 / CH;
    const int* tw = (const int*)(smem + L.slot0 + s * L.slot_bytes);
    const int m0 = lane / CH; // row within a copy
    int r1[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; i++) r1[i] = EXACT || R.c0 + i < R.c1 ? tw[(R.c0 + i) * RPC + m0] & kRowMask : 0;
#pragma unroll
    for (int i = 0; i < MAXC; i++)
        off[i] = (uint32_t)(r1[i] == 0 ? 0 : r1[i] - 1) * (uint32_t)g.row +
                 copy_chunk<D>((R.c0 + i) * RPC + m0, lane) * 8;
}

// EXACT: the wave issues exactly MAXC copies (the copies divide evenly among
// the loader waves), so no copy is conditional.
template <int D, int MAXC, bool EXACT>
__device__ inline void stream_issue(LoaderRange R, int hh, const uint32_t (&off)[MAXC],
                                    const uint16_t* __restrict__ src, unsigned char* dst) {
    const uint16_t* sh = src + hh * D;
#pragma unroll
    for (int i = 0; i < MAXC; i++)
        if (EXACT || R.c0 + i < R.c1)
            __builtin_amdgcn_global_load_lds((const void*)(sh + off[i]), (lds_void*)(dst + (R.c0 + i) * 1024), 16, 0,
                                             kNonTemporal);
}

// K and Q of a unit of head hh (source offsets off from its table) into
// buffer pair b, and for loader 0 the streamed bias slice into bias slot s.
template <int D, int MAXC, bool EXACT>
__device__ inline void stream_copy_kq(const Geometry& g, const StreamLds& L, unsigned char* smem, int j,
                                      LoaderRange R, int lane, int hh, const uint32_t (&off)[MAXC], int s, int b,
                                      const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                      const float* __restrict__ table) {
    stream_issue<D, MAXC, EXACT>(R, hh, off, k, smem + L.k0 + b * L.tb);
    stream_issue<D, MAXC, EXACT>(R, hh, off, q, smem + L.q0 + b * L.tb);
    if (j == 0 && !L.bias_resident) {
        float* bdst = (float*)(smem + L.bias) + s * L.TSP;
        for (int jj = 0; jj * 64 < L.TSP; jj++) {
            const int i = jj * 64 + lane;
            const float* src = table + (i < g.table_size ? i * g.heads + hh : 0);
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(bdst + jj * 64), 4, 0, 0);
        }
    }
}

// What a compute wave carries from the first half of a unit to the second.
template <int KT>
struct TileState {
    unsigned pk[KT][2]; // bf16 P: 4 keys per tile in two dwords
    int n, r;           // query index in the window; its source row (or -1)
    float mc;           // the exponents' reference (the row max, log2 units)
};

// Byte offsets, within a head's bias slice, of the biases a lane adds: they
// depend only on the positions of its query and keys inside the window, so a
// compute wave computes them once.  With BIAS_VEC the 4 keys of a lane are
// neighbours in one window row and one offset (of the lowest of 4 consecutive
// entries) serves them; otherwise there is one offset per key.
template <int KT_FIXED, bool BIAS_VEC>
struct BiasOffsets {
    int off[(KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles)][BIAS_VEC ? 1 : 4];
};

template <int KT_FIXED, bool BIAS_VEC>
__device__ inline void bias_offsets(const Geometry& g, const StreamLds& L, const unsigned char* smem, int qt,
                                    int lane, BiasOffsets<KT_FIXED, BIAS_VEC>& bo) {
    constexpr int KB = KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles;
    const int col = lane & 15, grp = lane >> 4;
    const int* kb4 = (const int*)(smem + L.kb4);
    const int n = qt * 16 + col;
    int qb4;
    if (n < g.N) {
        int lt, ly, lx;
        local_coords(g, n, lt, ly, lx);
        qb4 = (((lt * g.tdy + ly) * g.tdx + lx) + g.c0) * 4;
    } else {
        qb4 = (g.table_size - 1) * 4; // largest qb keeps qb - kb inside the table
    }
#pragma unroll
    for (int kt = 0; kt < KB; kt++) {
        const int key0 = kt * 16 + grp * 4; // kb4 has NP entries, padded keys included
        if (KT_FIXED == 0 && key0 >= L.NP) {
#pragma unroll
            for (int i = 0; i < (BIAS_VEC ? 1 : 4); i++) bo.off[kt][i] = 0;
        } else if (BIAS_VEC) {
            bo.off[kt][0] = qb4 - kb4[key0] - 12; // entries qb - kb0 - 3 .. qb - kb0
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) bo.off[kt][i] = qb4 - kb4[key0 + i];
        }
    }
}

// First half of unit uu for this wave's tile qt: S^T = K Q^T, logits, mask and
// softmax, from K, Q in buffer b and the table in slot s.
template <int D, int KT_FIXED, bool BIAS_VEC>
__device__ inline void stream_qk(const Geometry& g, const StreamLds& L, const unsigned char* smem, int qt, int lane,
                                 uint32_t uu, int s, int b, const BiasOffsets<KT_FIXED, BIAS_VEC>& bo,
                                 TileState<(KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles)>& ts) {
    constexpr int KSTEPS = D / 32;
    constexpr int KB = KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles;
    const int col = lane & 15, grp = lane >> 4;
    const int N = g.N;
    const int KT = KT_FIXED > 0 ? KT_FIXED : L.NP / 16;
    const Unit U = decode_unit(g, uu);
    const bool masked_window = window_maybe_masked(g, U.wc);
    const int* tw = (const int*)(smem + L.slot0 + s * L.slot_bytes);
    const uint16_t* Ks = (const uint16_t*)(smem + L.k0 + b * L.tb);
    const uint16_t* Qs = (const uint16_t*)(smem + L.q0 + b * L.tb);
    const unsigned char* bias_bytes = smem + L.bias + (size_t)(L.bias_resident ? U.h : s) * L.TSP * 4;
    const int n = qt * 16 + col;
    const int qword = tw[n];
    const int qreg = (unsigned)qword >> 28;
    ts.n = n;
    ts.r = (qword & kRowMask) - 1;
    float bias[KB][4]; // read tile by tile, after the products (addresses need no LDS reads)
    bf16x8 qf[KSTEPS]; // B operand: query n, d = 32 ks + 8 grp + 0..7
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++)
        qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Qs + n * D + k_slot<D>(n, ks * 4 + grp) * 8));
    f32x4 sc[KB];
#pragma unroll
    for (int kt = 0; kt < KB; kt++) {
        if (KT_FIXED > 0 || kt < KT) {
            const int krow = kt * 16 + col;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) {
                const bf16x8 a =
                    __builtin_bit_cast(bf16x8, *(const u32x4*)(Ks + krow * D + k_slot<D>(krow, ks * 4 + grp) * 8));
                acc = mfma32(a, qf[ks], acc);
            }
            sc[kt] = acc;
        }
    }
#pragma unroll
    for (int kt = 0; kt < KB; kt++) {
        if (KT_FIXED > 0 || kt < KT) {
            if (BIAS_VEC) {
                const float* bp = (const float*)(bias_bytes + bo.off[kt][0]);
                bias[kt][3] = bp[0];
                bias[kt][2] = bp[1];
                bias[kt][1] = bp[2];
                bias[kt][0] = bp[3];
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++) bias[kt][i] = *(const float*)(bias_bytes + bo.off[kt][i]);
            }
            // logits, natural units: scale * q.k + bias
            sc[kt] = f32x4{fmaf(sc[kt][0], g.scale, bias[kt][0]), fmaf(sc[kt][1], g.scale, bias[kt][1]),
                           fmaf(sc[kt][2], g.scale, bias[kt][2]), fmaf(sc[kt][3], g.scale, bias[kt][3])};
        } else {
            sc[kt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
    }
    // the mask, on windows that can hold hidden keys (all tiles) or whose last
    // tile runs past N (that tile only); a separate loop, so that windows
    // without hidden keys read no mask words at all
    if (masked_window || KT * 16 > N) {
#pragma unroll
        for (int kt = 0; kt < KB; kt++) {
            const int key0 = kt * 16;
            if ((KT_FIXED > 0 || kt < KT) && (masked_window || key0 + 16 > N)) {
                const int4 kr4 = *(const int4*)(tw + key0 + grp * 4);
                sc[kt][0] = ((unsigned)kr4.x >> 28) == (unsigned)qreg ? sc[kt][0] : -INFINITY;
                sc[kt][1] = ((unsigned)kr4.y >> 28) == (unsigned)qreg ? sc[kt][1] : -INFINITY;
                sc[kt][2] = ((unsigned)kr4.z >> 28) == (unsigned)qreg ? sc[kt][2] : -INFINITY;
                sc[kt][3] = ((unsigned)kr4.w >> 28) == (unsigned)qreg ? sc[kt][3] : -INFINITY;
            }
        }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KB; kt++)
        bmax = fmaxf(bmax, fmaxf(fmaxf(sc[kt][0], sc[kt][1]), fmaxf(sc[kt][2], sc[kt][3])));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mc = (bmax == -INFINITY ? 0.f : bmax) * kLog2e;
    ts.mc = mc;
#pragma unroll
    for (int kt = 0; kt < KB; kt++) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[kt][i], kLog2e, -mc));
        ts.pk[kt][0] = pack_bf16x2(p[0], p[1]);
        ts.pk[kt][1] = pack_bf16x2(p[2], p[3]);
    }
}

// Second half: O^T = V^T P^T from V in buffer b, divide by the sum and leave
// the O tile in this tile's rows of the LDS staging buffer (the loader waves
// store it).  With lse, each real query's log-sum-exp of its logits goes to
// lse[row * heads + hh] (natural log), from the reference and the row sum.
template <int D, int KT_FIXED>
__device__ inline void stream_pv(const StreamLds& L, unsigned char* smem, int lane, int b,
                                 const TileState<(KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles)>& ts,
                                 float* __restrict__ lse = nullptr, int hh = 0, int heads = 0) {
    constexpr int DT = D / 16;
    constexpr int KB = KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles;
    const int col = lane & 15, grp = lane >> 4;
    const int KT = KT_FIXED > 0 ? KT_FIXED : L.NP / 16;
    const unsigned one2 = 0x3F803F80u; // two bf16 ones
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});
    const unsigned char* Vb = smem + L.v0 + b * L.tb;
    uint16_t* Os = (uint16_t*)(smem + L.o0);
    f32x4 o[DT], osum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // V^T fragment of key tile t: lane (col, grp) gets keys 16t + 4grp + 0..3 at
    // d = 16 dt + col; lane s of the group points at row 16t + 4grp + s/4, d 16dt + 4(s%4)
    auto vt_frag = [&](int t0, int dt) __attribute__((always_inline)) {
        const int row = t0 * 16 + grp * 4 + (col >> 2);
        const int d = dt * 16 + (col & 3) * 4;
        const unsigned char* p = Vb + row * (D * 2) + k_slot<D>(row, d >> 3) * 16 + (d & 7) * 2;
        const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_void*)p);
        return __builtin_bit_cast(u32x2, x);
    };
#pragma unroll
    for (int kt = 0; kt < KB; kt += 2) {
        const bool pair = kt + 1 < KB && (KT_FIXED > 0 || kt + 1 < KT);
        if (pair) {
            const bf16x8 bop =
                __builtin_bit_cast(bf16x8, u32x4{ts.pk[kt][0], ts.pk[kt][1], ts.pk[kt + 1][0], ts.pk[kt + 1][1]});
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const u32x2 lo = vt_frag(kt, dt);
                const u32x2 hi = vt_frag(kt + 1, dt);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                o[dt] = mfma32(a, bop, o[dt]);
            }
            osum = mfma32(ones8, bop, osum);
        } else if (KT_FIXED > 0 || kt < KT) {
            // a lone last tile: the same 32-deep product with the second key
            // tile's slots zero, so every accumulation chain uses one opcode
            const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{ts.pk[kt][0], ts.pk[kt][1], 0u, 0u});
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const u32x2 lo = vt_frag(kt, dt);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], 0u, 0u});
                o[dt] = mfma32(a, bop, o[dt]);
            }
            osum = mfma32(ones8, bop, osum);
        }
    }
    // O tile into the staging rows of this tile (same swizzle)
    const int n = ts.n;
    const float inv = ts.r >= 0 ? __builtin_amdgcn_rcpf(osum[0]) : 0.f;
    if (lse != nullptr && ts.r >= 0 && grp == 0)
        lse[(uint64_t)(uint32_t)ts.r * (uint32_t)heads + hh] = (ts.mc + log2f(osum[0])) * kLn2;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
        const u32x2 w = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv), pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
        const int c = dt * 2 + (grp >> 1); // 16-byte chunk of d = 16 dt + 4 grp
        *(u32x2*)(Os + n * D + k_slot<D>(n, c) * 8 + (grp & 1) * 4) = w;
    }
}

// Rows of one batch item in the tensors the streaming schedule reads and
// writes (real-token layout, or window-major when staged), and its bytes.
__host__ __device__ inline uint64_t stream_item_rows(const Geometry& g, bool staged) {
    return staged ? (uint64_t)g.nW * g.N : (uint64_t)g.ext[0] * g.ext[1] * g.ext[2];
}
__host__ __device__ inline uint64_t stream_item_bytes(const Geometry& g, bool staged) {
    return stream_item_rows(g, staged) * (uint64_t)g.row * 2;
}

// Loader j's stores of a unit's O (table in slot s) from the LDS staging
// buffer: whole 128-byte token rows of its own row range, to the real token or,
// in the staged layout, also to pad slots (zeros); other lanes store out of
// range, which the buffer range check drops.  The buffer resource starts at
// the unit's batch item, so offsets stay below 2^31 whatever the batch.
template <int D, int MAXC, bool EXACT>
__device__ inline void stream_store_o(const Geometry& g, const StreamLds& L, const unsigned char* smem,
                                      uint16_t* __restrict__ out, LoaderRange R, int lane, uint32_t uu, int s,
                                      int staged) {
    constexpr int CH = D / 8;
    constexpr int RPC = 64 / CH;
    const int* tw = (const int*)(smem + L.slot0 + s * L.slot_bytes);
    const uint16_t* Os = (const uint16_t*)(smem + L.o0);
    const Unit U = decode_unit(g, uu);
    const uint64_t item_rows = stream_item_rows(g, staged);
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(out + (uint64_t)U.b * item_rows * (uint32_t)g.row), 0, (int)stream_item_bytes(g, staged), kBufferWord3);
    const int row0 = (int)((uint64_t)U.b * item_rows); // first row of the batch item
    const int c = lane % CH;
    u32x4 val[MAXC];
    int rm[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
        const int m = (R.c0 + i) * RPC + lane / CH;
        if (EXACT || R.c0 + i < R.c1) {
            val[i] = *(const u32x4*)(Os + m * D + k_slot<D>(m, c) * 8);
            rm[i] = (tw[m] & kRowMask) - 1;
        }
    }
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
        if (EXACT || R.c0 + i < R.c1) {
            const int m = (R.c0 + i) * RPC + lane / CH;
            const int orow = rm[i] >= 0 ? rm[i] : (staged && m < g.N ? (int)(U.wi * (uint32_t)g.N + m) : -1);
            const uint32_t ob =
                orow >= 0 ? ((uint32_t)(orow - row0) * (uint32_t)g.row + U.h * D + c * 8) * 2 : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(val[i], ors, ob, 0, kNonTemporal);
        }
    }
}


} // namespace swa
