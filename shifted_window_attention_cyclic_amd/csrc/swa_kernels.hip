// HIP kernels for shifted-window multi-head self-attention on gfx950.
//
// The forward pass computed here is the window (Swin) attention with
// shifted-window execution described on the TERRA page (abstract: tokens are
// routed from the spatial layout into window layouts for the Transformer and
// back; Fig. 5 caption: shift token routes; Table I: padded resolution; Table
// V: heads and window size).  Kernels:
//   gather_kernel      spatial layout -> window-major layout (pad, roll, partition)
//   scatter_kernel     window-major layout -> spatial layout (reverse)
//   visibility_kernel  the attention mask of one window, as the kernels use it
//   attn_f32_kernel    fp32 window attention (VALU), one block per (window, head)
//   attn_bf16_kernel   bf16 window attention on MFMA with fp32 accumulation and
//                      softmax; reads Q/K/V straight from the spatial layout and
//                      writes O back to it (fused), or works on window-major
//                      buffers (staged)
#include <hip/hip_runtime.h>
#include <math.h>
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

// --------------------------------------------------------------------------
// gather / scatter: one team of kTeam threads per token row, 16-byte chunks.
// --------------------------------------------------------------------------
constexpr int kTeam = 8;

__global__ __launch_bounds__(256) void gather_kernel(Geometry g, int row_chunks,
                                                     const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst) {
    const int64_t slots = g.windows * g.N;
    const int64_t team0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
    const int lane = threadIdx.x % kTeam;
    const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
    for (int64_t slot = team0; slot < slots; slot += teams) {
        int64_t wi = slot / g.N;
        int n = (int)(slot - wi * g.N);
        int b, wc[3];
        window_coords(g, wi, b, wc);
        TokenInfo ti = token_info(g, b, wc, n);
        u32x4* d = dst + slot * row_chunks;
        if (ti.tok < 0) {
            for (int c = lane; c < row_chunks; c += kTeam) d[c] = u32x4{0, 0, 0, 0};
        } else {
            const u32x4* s = src + ti.tok * row_chunks;
            for (int c = lane; c < row_chunks; c += kTeam) d[c] = s[c];
        }
    }
}

__global__ __launch_bounds__(256) void scatter_kernel(Geometry g, int row_chunks,
                                                      const u32x4* __restrict__ src,
                                                      u32x4* __restrict__ dst) {
    const int64_t tokens = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    const int64_t team0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
    const int lane = threadIdx.x % kTeam;
    const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
    for (int64_t tok = team0; tok < tokens; tok += teams) {
        int64_t r = tok;
        int c[3];
        c[2] = (int)(r % g.ext[2]);
        r /= g.ext[2];
        c[1] = (int)(r % g.ext[1]);
        r /= g.ext[1];
        c[0] = (int)(r % g.ext[0]);
        int b = (int)(r / g.ext[0]);
        // rolled coordinate c' = (c - s) mod P; window c' / w, local c' % w
        int64_t wi = b;
        int n = 0;
        for (int a = 0; a < 3; a++) {
            int cr = c[a] - g.shift[a];
            if (cr < 0) cr += g.pad[a];
            wi = wi * g.nwin[a] + cr / g.win[a];
            n = n * g.win[a] + cr % g.win[a];
        }
        const u32x4* s = src + (wi * g.N + n) * row_chunks;
        u32x4* d = dst + tok * row_chunks;
        for (int k = lane; k < row_chunks; k += kTeam) d[k] = s[k];
    }
}

static int copy_blocks(int64_t teams) {
    int64_t blocks = (teams * kTeam + 255) / 256;
    const int64_t cap = 256 * 64; // enough to fill the chip; the kernels loop
    return (int)(blocks < cap ? (blocks < 1 ? 1 : blocks) : cap);
}

hipError_t launch_gather(const Geometry& g, int elem_bytes, const void* src, void* dst,
                         hipStream_t s) {
    int row_chunks = g.row * elem_bytes / 16;
    hipLaunchKernelGGL(gather_kernel, dim3(copy_blocks(g.windows * g.N)), dim3(256), 0, s, g,
                       row_chunks, (const u32x4*)src, (u32x4*)dst);
    return hipGetLastError();
}

hipError_t launch_scatter(const Geometry& g, int elem_bytes, const void* src, void* dst,
                          hipStream_t s) {
    int row_chunks = g.row * elem_bytes / 16;
    int64_t tokens = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    hipLaunchKernelGGL(scatter_kernel, dim3(copy_blocks(tokens)), dim3(256), 0, s, g, row_chunks,
                       (const u32x4*)src, (u32x4*)dst);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// visibility export
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void visibility_kernel(Geometry g, int64_t wi,
                                                         uint8_t* __restrict__ out) {
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= g.N * g.N) return;
    int n = idx / g.N, m = idx % g.N;
    int b, wc[3];
    window_coords(g, wi, b, wc);
    int qw = query_word(token_info(g, b, wc, n));
    int kw = key_word(token_info(g, b, wc, m));
    out[idx] = visible(qw, kw) ? 1 : 0;
}

hipError_t launch_visibility(const Geometry& g, int64_t window, uint8_t* out, hipStream_t s) {
    int total = g.N * g.N;
    hipLaunchKernelGGL(visibility_kernel, dim3((total + 255) / 256), dim3(256), 0, s, g, window,
                       out);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Per-window token tables in LDS, shared by both attention kernels:
//   kword[m], qword[n]  mask words (see swa_geometry.h)
//   rowi[n]             row index of token n in the tensors read and written:
//                       the real token index (fused) or window*N + n (staged);
//                       -1 for pad tokens and slots past N
// --------------------------------------------------------------------------
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

// --------------------------------------------------------------------------
// fp32 attention: one block per (window, head), one thread per query, online
// softmax over the window's keys held in LDS.
// --------------------------------------------------------------------------
constexpr int kF32Threads = 256;

__host__ __device__ inline size_t f32_lds_bytes(const Geometry& g) {
    return (size_t)g.N * g.head_dim * 2 * sizeof(float) + (size_t)g.table_size * sizeof(float) +
           (size_t)g.N * 3 * sizeof(int);
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(Geometry g, int staged,
                                                               const float* __restrict__ q,
                                                               const float* __restrict__ k,
                                                               const float* __restrict__ v,
                                                               const float* __restrict__ table,
                                                               float* __restrict__ out) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int N = g.N;
    float* Ks = (float*)smem;
    float* Vs = Ks + N * D;
    float* bias = Vs + N * D;
    int* kword = (int*)(bias + g.table_size);
    int* qword = kword + N;
    int* rowi = qword + N;

    const int64_t total = g.windows * g.heads;
    const int64_t work = xcd_work_index(blockIdx.x, total);
    const int64_t wi = work / g.heads;
    const int h = (int)(work - wi * g.heads);

    fill_token_tables(g, wi, staged != 0, N, kword, qword, rowi);
    for (int i = threadIdx.x; i < g.table_size; i += blockDim.x)
        bias[i] = table[(int64_t)i * g.heads + h];
    __syncthreads();
    for (int i = threadIdx.x; i < N * D; i += blockDim.x) {
        int m = i / D, e = i % D;
        int r = rowi[m];
        float kv = 0.f, vv = 0.f;
        if (r >= 0) {
            int64_t off = (int64_t)r * g.row + (int64_t)h * D + e;
            kv = k[off];
            vv = v[off];
        }
        Ks[i] = kv;
        Vs[i] = vv;
    }
    __syncthreads();

    for (int n = threadIdx.x; n < N; n += blockDim.x) {
        int r = rowi[n];
        int qw = qword[n];
        if (r < 0) {
            if (staged) {
                float* o = out + ((wi * N + n) * (int64_t)g.row + (int64_t)h * D);
                for (int e = 0; e < D; e++) o[e] = 0.f;
            }
            continue;
        }
        float qv[D], acc[D];
        const float* qp = q + (int64_t)r * g.row + (int64_t)h * D;
        for (int e = 0; e < D; e++) {
            qv[e] = qp[e];
            acc[e] = 0.f;
        }
        float mx = -INFINITY, den = 0.f;
        for (int m = 0; m < N; m++) {
            int kw = kword[m];
            if (!visible(qw, kw)) continue;
            float dot = 0.f;
            for (int e = 0; e < D; e++) dot = fmaf(qv[e], Ks[m * D + e], dot);
            float s = dot * g.scale + bias[(qw & 0xFFFF) - (kw & 0xFFFF)];
            if (s > mx) {
                float alpha = expf(mx - s); // 0 on the first visible key
                den *= alpha;
                for (int e = 0; e < D; e++) acc[e] *= alpha;
                mx = s;
            }
            float p = expf(s - mx);
            den += p;
            for (int e = 0; e < D; e++) acc[e] = fmaf(p, Vs[m * D + e], acc[e]);
        }
        float inv = 1.f / den;
        float* o = out + (int64_t)r * g.row + (int64_t)h * D;
        for (int e = 0; e < D; e++) o[e] = acc[e] * inv;
    }
}

hipError_t launch_attention_f32(const Geometry& g, bool staged, const float* q, const float* k,
                                const float* v, const float* table, float* out, hipStream_t s) {
    size_t lds = f32_lds_bytes(g);
    dim3 grid((unsigned)(g.windows * g.heads));
    if (g.head_dim == 32)
        hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(kF32Threads), lds, s, g, (int)staged, q,
                           k, v, table, out);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kF32Threads), lds, s, g, (int)staged, q,
                           k, v, table, out);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// bf16 attention on MFMA.
//
// Block = (window, head), 4 waves.  K of the window goes to LDS as [key][d];
// V goes to LDS transposed, [d][key], so the PV product can read 4 keys of
// one d-row with one 8-byte load.  Each wave takes query tiles of 16 queries
// and computes, per tile:
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS,
//                 B = Q rows straight from global memory); lane l then holds
//                 scores of query (l % 16) against keys 4*(l/16) + 0..3 of
//                 every 16-key tile,
//   bias + mask   from LDS tables, in base-2 units (scaled by log2 e),
//   softmax       online over blocks of kKeyTilesPerBlock key tiles: running
//                 max and sum per query, reduced across the 4 lanes that share
//                 a query,
//   O^T = V^T P^T with the same MFMA (A = V^T from LDS, B = bf16 P straight
//                 from the score registers: two 16-key tiles give the 8 keys
//                 of one 32-deep step; an odd last tile uses 16x16x16),
//   epilogue      divide by the sum, round to bf16, store 4 d-values per lane.
// Both products use the same key order on both operands, so any order of
// the 32 reduction slots the hardware uses gives the same sums.
// --------------------------------------------------------------------------
constexpr int kBf16Waves = 4;
constexpr int kKeyTilesPerBlock = 9;

struct Bf16Lds {
    int NP, KSTR, VSTR;
    size_t ks, vt, bias, kword, qword, rowi, total;
};

__host__ __device__ inline Bf16Lds bf16_lds(const Geometry& g) {
    Bf16Lds L;
    L.NP = (g.N + 15) / 16 * 16;
    L.KSTR = g.head_dim + 8; // bf16 elements per K row (16-byte pad against bank conflicts)
    L.VSTR = L.NP + 4;       // bf16 elements per V^T row
    L.ks = 0;
    L.vt = L.ks + (size_t)L.NP * L.KSTR * 2;
    L.bias = L.vt + (size_t)g.head_dim * L.VSTR * 2;
    L.bias = (L.bias + 15) / 16 * 16;
    L.kword = L.bias + (size_t)g.table_size * 4;
    L.qword = L.kword + (size_t)L.NP * 4;
    L.rowi = L.qword + (size_t)L.NP * 4;
    L.total = L.rowi + (size_t)L.NP * 4;
    return L;
}

__device__ inline bf16x8 load_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *(const u32x4*)p);
}

__device__ inline unsigned pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (unsigned)__builtin_bit_cast(uint16_t, x) | ((unsigned)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D>
__global__ __launch_bounds__(kBf16Waves * 64) void attn_bf16_kernel(
    Geometry g, int staged, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ table, uint16_t* __restrict__ out) {
    constexpr int KSTEPS = D / 32; // 32-deep steps of Q K^T
    constexpr int DT = D / 16;     // 16-row d tiles of O^T
    constexpr int CH = D / 8;      // 16-byte chunks per (token, head)
    constexpr int KB = kKeyTilesPerBlock;
    extern __shared__ __align__(16) unsigned char smem[];
    const Bf16Lds L = bf16_lds(g);
    uint16_t* Ks = (uint16_t*)(smem + L.ks);
    uint16_t* Vt = (uint16_t*)(smem + L.vt);
    float* bias = (float*)(smem + L.bias);
    int* kword = (int*)(smem + L.kword);
    int* qword = (int*)(smem + L.qword);
    int* rowi = (int*)(smem + L.rowi);
    const int N = g.N, NP = L.NP, KT = NP / 16;

    const int64_t total = g.windows * g.heads;
    const int64_t work = xcd_work_index(blockIdx.x, total);
    const int64_t wi = work / g.heads;
    const int h = (int)(work - wi * g.heads);

    fill_token_tables(g, wi, staged != 0, NP, kword, qword, rowi);
    for (int i = threadIdx.x; i < g.table_size; i += blockDim.x)
        bias[i] = table[(int64_t)i * g.heads + h] * kLog2e;
    __syncthreads();

    // K rows and V^T columns into LDS; pad keys are zeros (their P is 0, and
    // 0 * 0 keeps the PV sums finite).
    for (int i = threadIdx.x; i < NP * CH; i += blockDim.x) {
        int m = i / CH, c = i % CH;
        int r = rowi[m];
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (r >= 0) {
            int64_t off = (int64_t)r * g.row + (int64_t)h * D + c * 8;
            kv = *(const u32x4*)(k + off);
            vv = *(const u32x4*)(v + off);
        }
        *(u32x4*)(Ks + m * L.KSTR + c * 8) = kv;
        for (int j = 0; j < 4; j++) {
            Vt[(c * 8 + 2 * j) * L.VSTR + m] = (uint16_t)(vv[j] & 0xFFFF);
            Vt[(c * 8 + 2 * j + 1) * L.VSTR + m] = (uint16_t)(vv[j] >> 16);
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const float sl2 = g.scale * kLog2e;

    for (int qt = wave; qt < KT; qt += kBf16Waves) {
        const int n = qt * 16 + col;
        const int qw = qword[n];
        const int qb = qw & 0xFFFF;
        const int r = rowi[n];
        bf16x8 qop[KSTEPS];
        for (int ks = 0; ks < KSTEPS; ks++) {
            if (r >= 0)
                qop[ks] = load_bf16x8(q + (int64_t)r * g.row + (int64_t)h * D + ks * 32 + grp * 8);
            else
                qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
        f32x4 o[DT];
        for (int dt = 0; dt < DT; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float mrun = -INFINITY, lsum = 0.f;

        for (int kb0 = 0; kb0 < KT; kb0 += KB) {
            float s[KB][4];
            float bmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KB; kt++) {
                if (kb0 + kt < KT) {
                    const int key0 = (kb0 + kt) * 16;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ks++) {
                        bf16x8 a = load_bf16x8(Ks + (key0 + col) * L.KSTR + ks * 32 + grp * 8);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[ks], acc, 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        int kw = kword[key0 + grp * 4 + i];
                        float val = acc[i] * sl2 + bias[qb - (kw & 0xFFFF)];
                        val = visible(qw, kw) ? val : -INFINITY;
                        s[kt][i] = val;
                        bmax = fmaxf(bmax, val);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) s[kt][i] = -INFINITY;
                }
            }
            bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
            bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
            const float mnew = fmaxf(mrun, bmax);
            const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrun - msafe);
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) o[dt] *= alpha;
            mrun = mnew;

            unsigned pk[KB][2]; // bf16 P, 4 keys per tile packed in two dwords
#pragma unroll
            for (int kt = 0; kt < KB; kt++) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    p[i] = __builtin_amdgcn_exp2f(s[kt][i] - msafe);
                    lsum += p[i];
                }
                pk[kt][0] = pack_bf16x2(p[0], p[1]);
                pk[kt][1] = pack_bf16x2(p[2], p[3]);
            }

#pragma unroll
            for (int kt = 0; kt < KB; kt += 2) {
                const int t0 = kb0 + kt;
                if (kt + 1 < KB && t0 + 1 < KT) {
                    bf16x8 b = __builtin_bit_cast(
                        bf16x8, u32x4{pk[kt][0], pk[kt][1], pk[kt + 1][0], pk[kt + 1][1]});
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const uint16_t* vr = Vt + (dt * 16 + col) * L.VSTR + t0 * 16 + grp * 4;
                        u32x2 lo = *(const u32x2*)vr;
                        u32x2 hi = *(const u32x2*)(vr + 16);
                        bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, o[dt], 0, 0, 0);
                    }
                } else if (t0 < KT) {
                    i16x4 b = __builtin_bit_cast(i16x4, u32x2{pk[kt][0], pk[kt][1]});
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const uint16_t* vr = Vt + (dt * 16 + col) * L.VSTR + t0 * 16 + grp * 4;
                        i16x4 a = __builtin_bit_cast(i16x4, *(const u32x2*)vr);
                        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, o[dt], 0, 0, 0);
                    }
                }
            }
        }
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);

        int64_t orow = r;
        if (r < 0 && staged) orow = wi * N + n; // staged: pad slots of O are written as zeros
        if (orow >= 0 && n < N) {
            const float inv = r >= 0 ? 1.f / lsum : 0.f;
            uint16_t* op = out + orow * g.row + (int64_t)h * D + grp * 4;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                u32x2 w = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                           pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
                *(u32x2*)(op + dt * 16) = w;
            }
        }
    }
}

size_t attention_lds_bytes(const Geometry& g, bool bf16) {
    return bf16 ? bf16_lds(g).total : f32_lds_bytes(g);
}

hipError_t launch_attention_bf16(const Geometry& g, bool staged, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const float* table,
                                 uint16_t* out, hipStream_t s) {
    size_t lds = bf16_lds(g).total;
    dim3 grid((unsigned)(g.windows * g.heads));
    if (g.head_dim == 32)
        hipLaunchKernelGGL(attn_bf16_kernel<32>, grid, dim3(kBf16Waves * 64), lds, s, g,
                           (int)staged, q, k, v, table, out);
    else
        hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kBf16Waves * 64), lds, s, g,
                           (int)staged, q, k, v, table, out);
    return hipGetLastError();
}

hipError_t prepare_kernels() {
    const int max_lds = 160 * 1024;
    hipError_t e;
    if ((e = hipFuncSetAttribute((const void*)attn_f32_kernel<32>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, max_lds)) != hipSuccess)
        return e;
    if ((e = hipFuncSetAttribute((const void*)attn_f32_kernel<64>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, max_lds)) != hipSuccess)
        return e;
    if ((e = hipFuncSetAttribute((const void*)attn_bf16_kernel<32>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, max_lds)) != hipSuccess)
        return e;
    return hipFuncSetAttribute((const void*)attn_bf16_kernel<64>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
}

} // namespace swa
