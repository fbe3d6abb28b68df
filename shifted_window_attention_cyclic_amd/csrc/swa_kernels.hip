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
//   attn_f32_kernel    fp32 window attention (VALU), one block per (window, head,
//                      32 queries), eight lanes per query
//   attn_bf16_stream_kernel
//                      bf16 window attention on MFMA with fp32 accumulation,
//                      windows of up to 9 query tiles: persistent workgroups,
//                      loader waves streaming each unit's K, Q, V through LDS
//                      while compute waves work on the one before
//   attn_bf16_kernel   the same arithmetic with one workgroup per (window,
//                      head): windows of up to 32 tiles, online softmax over
//                      9-tile key blocks, blocks masked for a whole query tile
//                      skipped
//   attn_bf16_kblock_kernel
//                      windows of any size: 256 queries per workgroup, K and V
//                      streamed in 32-key blocks, blocks masked for all of a
//                      wave's queries skipped
//   bias_head_major_kernel
//                      the head-major bias copy the key-blocked and per-unit
//                      kernels read
// Every bf16 kernel reads Q/K/V straight from the spatial layout and writes O
// back to it (fused), or works on window-major buffers (staged).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "swa_device.h"
#include "swa_geometry.h"
#include "swa_stream.h"

namespace swa {

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
// fp32 attention: one block per (window, head, block of 32 queries).  Each
// query takes kF32Split lanes; lane j runs an online softmax over the keys m
// with m % kF32Split == j (K and V rows from LDS, 16 bytes per read), and the
// lanes then merge their partial states (max, sum, weighted V) with
// shuffles.  So a 64-token window runs on two blocks of four busy waves,
// where a thread per query would leave three waves idle and run 64 keys in
// series.
// --------------------------------------------------------------------------
constexpr int kF32Threads = 256;
constexpr int kF32Split = 8;                        // lanes per query
constexpr int kF32Queries = kF32Threads / kF32Split; // queries per block

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
                                                               float* __restrict__ out,
                                                               float* __restrict__ lse) {
    static_assert(D % (4 * kF32Split) == 0, "rows read 16 bytes at a time, each lane writes 16-byte pieces of a row");
    extern __shared__ __align__(16) unsigned char smem[];
    const int N = g.N;
    float* Ks = (float*)smem;
    float* Vs = Ks + N * D;
    float* bias = Vs + N * D;
    int* kword = (int*)(bias + g.table_size);
    int* qword = kword + N;
    int* rowi = qword + N;

    // block -> (window, head, query block); the query blocks of a unit are
    // neighbours on one XCD and read its K and V from that XCD's L2
    const int QB = (N + kF32Queries - 1) / kF32Queries;
    const int64_t total = g.windows * g.heads * QB;
    const int64_t work = xcd_work_index(blockIdx.x, total);
    const int64_t unit = work / QB;
    const int qblk = (int)(work - unit * QB);
    const int64_t wi = unit / g.heads;
    const int h = (int)(unit - wi * g.heads);

    fill_token_tables(g, wi, staged != 0, N, kword, qword, rowi);
    for (int i = threadIdx.x; i < g.table_size; i += blockDim.x)
        bias[i] = table[(int64_t)i * g.heads + h];
    __syncthreads();
    for (int i = threadIdx.x; i < N * D / 4; i += blockDim.x) {
        const int m = i / (D / 4), e4 = i % (D / 4);
        const int r = rowi[m];
        float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (r >= 0) {
            const int64_t off = (int64_t)r * g.row + (int64_t)h * D + e4 * 4;
            kv = *(const float4*)(k + off);
            vv = *(const float4*)(v + off);
        }
        ((float4*)Ks)[i] = kv;
        ((float4*)Vs)[i] = vv;
    }
    __syncthreads();

    const int j = threadIdx.x % kF32Split; // this lane's keys: m % kF32Split == j
    {
        // the lanes of a query all run this (the shuffles need every one of them)
        const int n0 = qblk * kF32Queries + threadIdx.x / kF32Split;
        const int n = n0 < N ? n0 : N - 1;
        const int r = rowi[n];
        const int qw = qword[n];
        float qv[D], acc[D];
        const float* qp = q + (int64_t)(r < 0 ? 0 : r) * g.row + (int64_t)h * D;
#pragma unroll
        for (int e = 0; e < D; e += 4) {
            const float4 x = *(const float4*)(qp + e);
            qv[e] = x.x;
            qv[e + 1] = x.y;
            qv[e + 2] = x.z;
            qv[e + 3] = x.w;
        }
#pragma unroll
        for (int e = 0; e < D; e++) acc[e] = 0.f;
        float mx = -INFINITY, den = 0.f;
        for (int m = j; m < N; m += kF32Split) {
            const int kw = kword[m];
            if (!visible(qw, kw)) continue;
            const float4* kr = (const float4*)(Ks + m * D);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < D; e += 4) {
                const float4 x = kr[e / 4];
                dot = fmaf(qv[e], x.x, dot);
                dot = fmaf(qv[e + 1], x.y, dot);
                dot = fmaf(qv[e + 2], x.z, dot);
                dot = fmaf(qv[e + 3], x.w, dot);
            }
            const float sc = dot * g.scale + bias[(qw & 0xFFFF) - (kw & 0xFFFF)];
            if (sc > mx) {
                const float alpha = expf(mx - sc); // 0 on the first visible key
                den *= alpha;
#pragma unroll
                for (int e = 0; e < D; e++) acc[e] *= alpha;
                mx = sc;
            }
            const float p = expf(sc - mx);
            den += p;
            const float4* vr = (const float4*)(Vs + m * D);
#pragma unroll
            for (int e = 0; e < D; e += 4) {
                const float4 x = vr[e / 4];
                acc[e] = fmaf(p, x.x, acc[e]);
                acc[e + 1] = fmaf(p, x.y, acc[e + 1]);
                acc[e + 2] = fmaf(p, x.z, acc[e + 2]);
                acc[e + 3] = fmaf(p, x.w, acc[e + 3]);
            }
        }
        // merge the query's partial states: the common max, each part scaled to it
        float m4 = mx;
#pragma unroll
        for (int sh = 1; sh < kF32Split; sh <<= 1) m4 = fmaxf(m4, __shfl_xor(m4, sh));
        const float w = mx == -INFINITY ? 0.f : expf(mx - m4); // a lane that saw no visible key adds 0
        float d4 = den * w;
#pragma unroll
        for (int sh = 1; sh < kF32Split; sh <<= 1) d4 += __shfl_xor(d4, sh);
#pragma unroll
        for (int e = 0; e < D; e++) {
            float a = acc[e] * w;
#pragma unroll
            for (int sh = 1; sh < kF32Split; sh <<= 1) a += __shfl_xor(a, sh);
            acc[e] = a;
        }
        if (n0 >= N) return; // a query slot past the window: nothing to write
        if (r < 0) {         // pad query: no output (staged: its slot is zero)
            if (staged) {
                float* o = out + ((wi * N + n) * (int64_t)g.row + (int64_t)h * D);
#pragma unroll
                for (int e = 0; e < D / kF32Split; e++) o[j * (D / kF32Split) + e] = 0.f;
            }
            return;
        }
        const float inv = 1.f / d4;
        if (lse != nullptr && j == 0) lse[(int64_t)r * g.heads + h] = m4 + logf(d4);
        float* o = out + (int64_t)r * g.row + (int64_t)h * D;
        // lane j writes elements j D/kF32Split .. (j + 1) D/kF32Split - 1 (register indices stay static)
#pragma unroll
        for (int jj = 0; jj < kF32Split; jj++) {
            if (jj != j) continue;
#pragma unroll
            for (int e = 0; e < D / kF32Split; e += 4)
                *(float4*)(o + jj * (D / kF32Split) + e) =
                    float4{acc[jj * (D / kF32Split) + e] * inv, acc[jj * (D / kF32Split) + e + 1] * inv,
                           acc[jj * (D / kF32Split) + e + 2] * inv, acc[jj * (D / kF32Split) + e + 3] * inv};
        }
    }
}

hipError_t launch_attention_f32(const Geometry& g, bool staged, const float* q, const float* k,
                                const float* v, const float* table, float* out, float* lse, hipStream_t s) {
    size_t lds = f32_lds_bytes(g);
    dim3 grid((unsigned)(g.windows * g.heads * ((g.N + kF32Queries - 1) / kF32Queries)));
    if (g.head_dim == 32)
        hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(kF32Threads), lds, s, g, (int)staged, q,
                           k, v, table, out, lse);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kF32Threads), lds, s, g, (int)staged, q,
                           k, v, table, out, lse);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// bf16 attention on MFMA, per-unit schedule.
//
// Block = (window, head); wave w takes the 16-query tiles w, w + NWAVES, ...
// Phases:
//   A  the window's token table in LDS: one packed word per token (source row
//      + 1, 0 for pad, in bits 0..27; mask field in bits 28..31) and the bias
//      offset kb of every key (16 bits);
//   B  K and V of the window copied straight into LDS with global_load_lds
//      ([key][d], 16-byte chunks XOR-swizzled by row; a 1 KB copy moves 8
//      token rows of 128 bytes, every request a whole line), this head's bias
//      slice, and each wave's Q tiles into registers;
//   C  per 16-query tile of a wave:
//        S^T = K Q^T     v_mfma_f32_16x16x32_bf16, A = K from LDS, B = Q tile
//                        in registers, C = 0; lane l holds query (l % 16)
//                        against keys 4*(l/16) + 0..3 of every 16-key tile;
//        logits          scale * S + bias by one FMA; the bias of query n and
//                        key m sits at qb(n) - kb(m), and when the window's
//                        longitude extent is a multiple of 4 the 4 keys of a
//                        lane are neighbours in one window row, so their 4
//                        biases are 4 consecutive table entries;
//        mask            -inf where the key is pad, past N or on the other
//                        side of a masked wrap; only on windows / tiles that
//                        can hold such keys;
//        softmax         online over key blocks of up to 9 tiles:
//                        p = exp2(l*log2(e) - m*log2(e)), running max per query
//                        (reduced across the 4 lanes that share it);
//        O^T = V^T P^T   same MFMA, A = V^T fragments read with the transposing
//                        ds_read_b64_tr_b16, B = bf16 P straight from registers
//                        (two key tiles make one 32-deep step; an odd last tile
//                        is zero-extended); the row sum of the bf16 P comes from
//                        the same product with A = 1;
//        epilogue        divide by the sum, round to bf16, store 4 d-values
//                        per lane at the token's address.
// Both products use the same key order on both operands, so whatever order
// the hardware gives the 32 reduction slots the sums are the same.  The
// arithmetic is the streaming schedule's, so both give bit-identical outputs
// for windows that both take.  The kernel is specialised on the key-tile
// count of common window sizes (KT_FIXED > 0: straight-line code);
// KT_FIXED = 0 handles any count.
// --------------------------------------------------------------------------
constexpr int kKeyTilesPerBlock = 9;

struct Bf16Lds {
    int NP;
    size_t ks, vs, bias, tw, kb, total;
};

__host__ __device__ inline Bf16Lds bf16_lds(const Geometry& g) {
    Bf16Lds L;
    L.NP = (g.N + 15) / 16 * 16;
    L.ks = 0;
    L.vs = L.ks + (size_t)L.NP * g.head_dim * 2;
    L.bias = L.vs + (size_t)L.NP * g.head_dim * 2;
    L.tw = L.bias + ((size_t)g.table_size * 4 + 15) / 16 * 16;
    L.kb = L.tw + (size_t)L.NP * 4;
    L.total = L.kb + (size_t)L.NP * 2;
    return L;
}

template <int D, int NWAVES, int QT_MAX, int KT_FIXED, bool BIAS_VEC>
__global__ __launch_bounds__(NWAVES * 64) void attn_bf16_kernel(
    Geometry g, int staged, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ table, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int THREADS = NWAVES * 64;
    constexpr int KSTEPS = D / 32; // 32-deep steps of K Q^T
    constexpr int DT = D / 16;     // 16-row d tiles of O^T
    constexpr int CH = D / 8;      // 16-byte chunks per (token, head)
    constexpr int RPC = 64 / CH;   // token rows per 1 KB copy
    constexpr int KT_MAX = KT_FIXED > 0 ? KT_FIXED : NWAVES * QT_MAX;
    static_assert(KT_MAX <= NWAVES * QT_MAX, "every query tile needs a wave");
    constexpr int KB = (KT_FIXED > 0 && KT_FIXED <= kKeyTilesPerBlock) ? KT_FIXED : kKeyTilesPerBlock;
    static_assert(KT_FIXED == 0 || KT_FIXED % KB == 0, "fixed tile counts split into equal key blocks");
    constexpr int KB_UNROLL = KT_FIXED > 0 ? KT_FIXED / KB : 1;
    constexpr int BIAS_UNROLL = 4;
    extern __shared__ __align__(16) unsigned char smem[];
    const Bf16Lds L = bf16_lds(g);
    const uint16_t* Ks = (const uint16_t*)(smem + L.ks);
    const unsigned char* Vb = smem + L.vs;
    float* bias = (float*)(smem + L.bias);
    int* tw = (int*)(smem + L.tw);
    uint16_t* kb = (uint16_t*)(smem + L.kb);
    const int N = g.N, NP = L.NP;
    const int KT = KT_FIXED > 0 ? KT_FIXED : NP / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;

    // block -> (window, head); blocks are dealt to XCDs round-robin, so this
    // keeps the heads of a window and neighbouring windows on one XCD
    const uint32_t total = (uint32_t)(g.windows * g.heads);
    const uint32_t work = (uint32_t)xcd_work_index(blockIdx.x, total);
    const uint32_t wi = fdiv(g.fd_heads, work);
    const int h = (int)(work - wi * (uint32_t)g.heads);
    const int b = (int)fdiv(g.fd_nW, wi);
    int wc[3];
    {
        const uint32_t r = wi - (uint32_t)b * (uint32_t)g.nW;
        const uint32_t r2 = fdiv(g.fd_nwin2, r);
        wc[2] = (int)(r - r2 * (uint32_t)g.nwin[2]);
        wc[0] = (int)fdiv(g.fd_nwin1, r2);
        wc[1] = (int)(r2 - (uint32_t)wc[0] * (uint32_t)g.nwin[1]);
    }
    const bool masked_window = window_maybe_masked(g, wc);

    // ---- A: token table and key bias offsets
    for (int n = tid; n < NP; n += THREADS) {
        if (n < N) {
            int l[3];
            local_coords(g, n, l[0], l[1], l[2]);
            int region = 0, tok = b;
            bool is_pad = false;
#pragma unroll
            for (int a = 0; a < 3; a++) {
                const int cr = wc[a] * g.win[a] + l[a];
                int c = cr + g.shift[a];
                if (c >= g.pad[a]) c -= g.pad[a];
                is_pad |= c >= g.ext[a];
                if (!g.cyc[a] && cr >= g.pad[a] - g.shift[a]) region |= 1 << a;
                tok = tok * g.ext[a] + c;
            }
            const int row = is_pad ? -1 : (staged ? (int)(wi * (uint32_t)N + n) : tok);
            tw[n] = (row + 1) | ((region | (is_pad ? 8 : 0)) << 28);
            kb[n] = (uint16_t)((l[0] * g.tdy + l[1]) * g.tdx + l[2]);
        } else {
            tw[n] = 15 << 28;
            kb[n] = BIAS_VEC ? 3 : 0; // keeps qb - kb (- 3) inside the table
        }
    }
    __syncthreads();

    // ---- B: K and V copies into LDS (pad rows copy row 0: finite values that
    // get weight exactly 0), the bias slice, and each wave's Q tiles
    {
        const int ncopy = NP * CH / 64; // 1 KB copies per tensor
        const int m0 = lane / CH;
        for (int c = wave; c < 2 * ncopy; c += NWAVES) {
            const bool is_v = c >= ncopy;
            const int cc = is_v ? c - ncopy : c;
            const int ch = copy_chunk<D>(cc * RPC + m0, lane); // logical chunk landing in this lane's slot
            const int r1 = tw[cc * RPC + m0] & kRowMask;
            const uint64_t off = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + h * D + ch * 8;
            __builtin_amdgcn_global_load_lds((const void*)((is_v ? v : k) + off),
                                             (lds_void*)(smem + (is_v ? L.vs : L.ks) + cc * 1024), 16, 0, 0);
        }
    }
    bf16x8 qop[QT_MAX][KSTEPS];
#pragma unroll
    for (int t = 0; t < QT_MAX; t++) {
        const int qt = wave + t * NWAVES;
        const int r = qt < KT ? (tw[qt * 16 + col] & kRowMask) - 1 : -1;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            u32x4 val = {0, 0, 0, 0};
            if (r >= 0)
                val = *(const u32x4*)(q + (uint64_t)(uint32_t)r * (uint32_t)g.row + h * D + ks * 32 + grp * 8);
            qop[t][ks] = __builtin_bit_cast(bf16x8, val);
        }
    }
    for (int base = 0; base < g.table_size; base += BIAS_UNROLL * THREADS) {
        float bv[BIAS_UNROLL];
#pragma unroll
        for (int u = 0; u < BIAS_UNROLL; u++) {
            const int i = base + u * THREADS + tid;
            bv[u] = i < g.table_size ? table[(size_t)h * g.table_size + i] : 0.f; // head-major copy
        }
#pragma unroll
        for (int u = 0; u < BIAS_UNROLL; u++) {
            const int i = base + u * THREADS + tid;
            if (i < g.table_size) bias[i] = bv[u];
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); // this wave's LDS copies have landed
    __syncthreads();

    // ---- C: query tiles
    const unsigned one2 = 0x3F803F80u; // two bf16 ones
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});
    const unsigned char* bias_bytes = (const unsigned char*)bias;
    // Mask fields present in each key block, 16 bits per block.  A query sees a
    // key only when their fields are equal, so a key block that shares no field
    // with a query tile adds nothing to its output (P = 0) and leaves its
    // running max alone: it is skipped.  In a window split across a
    // non-cyclic boundary along time, a time slice of 12 x 12 tokens is exactly
    // one block of 9 tiles, so half of such a window's blocks drop out.
    constexpr int NKB = (KT_MAX + KB - 1) / KB;
    static_assert(NKB <= 4, "four 16-bit field sets in a 64-bit word");
    uint64_t ksets = ~(uint64_t)0;
    if (masked_window && NKB > 1) {
        ksets = 0;
#pragma unroll
        for (int bi = 0; bi < NKB; bi++) {
            unsigned m = 0;
            for (int kn = bi * KB * 16 + lane; kn < (bi + 1) * KB * 16 && kn < NP; kn += 64)
                m |= 1u << ((unsigned)tw[kn] >> 28);
#pragma unroll
            for (int sh = 32; sh >= 1; sh >>= 1) m |= __shfl_xor(m, sh);
            ksets |= (uint64_t)__builtin_amdgcn_readfirstlane(m) << (16 * bi);
        }
    }
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
    for (int t = 0; t < QT_MAX; t++) {
        const int qt = wave + t * NWAVES;
        if (qt >= KT) break;
        const int n = qt * 16 + col;
        const int qword = tw[n];
        const int qreg = (unsigned)qword >> 28;
        const int r = (qword & kRowMask) - 1;
        int qb4;
        if (n < N) {
            int lt, ly, lx;
            local_coords(g, n, lt, ly, lx);
            qb4 = (((lt * g.tdy + ly) * g.tdx + lx) + g.c0) * 4;
        } else {
            qb4 = (g.table_size - 1) * 4; // largest qb keeps qb - kb inside the table
        }
        const unsigned char* qbias = bias_bytes + qb4;
        // mask fields of the tile's 16 queries (one per lane column)
        unsigned qset = 1u << qreg;
#pragma unroll
        for (int sh = 8; sh >= 1; sh >>= 1) qset |= __shfl_xor(qset, sh);
        qset = __builtin_amdgcn_readfirstlane(qset);
        f32x4 o[DT], osum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float mrun = -INFINITY;

#pragma unroll KB_UNROLL
        for (int kb0 = 0; kb0 < (KT_FIXED > 0 ? KT_FIXED : KT); kb0 += KB) {
            if ((qset & (unsigned)(ksets >> (16 * (kb0 / KB)))) == 0) continue; // every pair masked
            f32x4 s[KB];
#pragma unroll
            for (int kt = 0; kt < KB; kt++) {
                const int key0 = (kb0 + kt) * 16;
                if (KT_FIXED > 0 || kb0 + kt < KT) {
                    const int krow = key0 + col;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ks++) {
                        const bf16x8 a = __builtin_bit_cast(
                            bf16x8, *(const u32x4*)(Ks + krow * D + k_slot<D>(krow, ks * 4 + grp) * 8));
                        acc = mfma32(a, qop[t][ks], acc);
                    }
                    s[kt] = acc;
                }
            }
            float bmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KB; kt++) {
                const int key0 = (kb0 + kt) * 16;
                if (KT_FIXED > 0 || kb0 + kt < KT) {
                    float bb[4];
                    if (BIAS_VEC) {
                        // keys key0 + 4*grp + i share a window row: biases at qb - kb0 - i
                        const float* bp = (const float*)(qbias - (int)kb[key0 + grp * 4] * 4) - 3;
                        bb[3] = bp[0];
                        bb[2] = bp[1];
                        bb[1] = bp[2];
                        bb[0] = bp[3];
                    } else {
                        const u32x2 kq = *(const u32x2*)(kb + key0 + grp * 4);
                        bb[0] = *(const float*)(qbias - (int)(kq[0] & 0xFFFF) * 4);
                        bb[1] = *(const float*)(qbias - (int)(kq[0] >> 16) * 4);
                        bb[2] = *(const float*)(qbias - (int)(kq[1] & 0xFFFF) * 4);
                        bb[3] = *(const float*)(qbias - (int)(kq[1] >> 16) * 4);
                    }
                    // logits, natural units: scale * q.k + bias
                    f32x4 lg = {fmaf(s[kt][0], g.scale, bb[0]), fmaf(s[kt][1], g.scale, bb[1]),
                                fmaf(s[kt][2], g.scale, bb[2]), fmaf(s[kt][3], g.scale, bb[3])};
                    if (masked_window || key0 + 16 > N) {
                        const int4 kr4 = *(const int4*)(tw + key0 + grp * 4);
                        lg[0] = ((unsigned)kr4.x >> 28) == (unsigned)qreg ? lg[0] : -INFINITY;
                        lg[1] = ((unsigned)kr4.y >> 28) == (unsigned)qreg ? lg[1] : -INFINITY;
                        lg[2] = ((unsigned)kr4.z >> 28) == (unsigned)qreg ? lg[2] : -INFINITY;
                        lg[3] = ((unsigned)kr4.w >> 28) == (unsigned)qreg ? lg[3] : -INFINITY;
                    }
                    s[kt] = lg;
                    bmax = fmaxf(bmax, fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
                } else {
                    s[kt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                }
            }
            bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
            bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
            const float mnew = fmaxf(mrun, bmax);
            const float mc = (mnew == -INFINITY ? 0.f : mnew) * kLog2e;
            if (kb0 > 0) { // rescale what earlier key blocks accumulated
                const float alpha = __builtin_amdgcn_exp2f(mrun * kLog2e - mc);
                osum *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; dt++) o[dt] *= alpha;
            }
            mrun = mnew;

            unsigned pk[KB][2]; // bf16 P: 4 keys per tile in two dwords
#pragma unroll
            for (int kt = 0; kt < KB; kt++) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(fmaf(s[kt][i], kLog2e, -mc));
                pk[kt][0] = pack_bf16x2(p[0], p[1]);
                pk[kt][1] = pack_bf16x2(p[2], p[3]);
            }

#pragma unroll
            for (int kt = 0; kt < KB; kt += 2) {
                const int t0 = kb0 + kt;
                const bool pair = kt + 1 < KB && (KT_FIXED > 0 || t0 + 1 < KT);
                if (pair) {
                    const bf16x8 bop = __builtin_bit_cast(
                        bf16x8, u32x4{pk[kt][0], pk[kt][1], pk[kt + 1][0], pk[kt + 1][1]});
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const u32x2 lo = vt_frag(t0, dt);
                        const u32x2 hi = vt_frag(t0 + 1, dt);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                        o[dt] = mfma32(a, bop, o[dt]);
                    }
                    osum = mfma32(ones8, bop, osum);
                } else if (KT_FIXED > 0 || t0 < KT) {
                    // a lone last tile: the same 32-deep product with the second key
                    // tile's slots zero (P = 0, V^T = 0), so every accumulation chain
                    // uses one MFMA opcode
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{pk[kt][0], pk[kt][1], 0u, 0u});
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const u32x2 lo = vt_frag(t0, dt);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], 0u, 0u});
                        o[dt] = mfma32(a, bop, o[dt]);
                    }
                    osum = mfma32(ones8, bop, osum);
                }
            }
        }

        int orow = r;
        if (r < 0 && staged) orow = (int)(wi * (uint32_t)N + n); // staged: pad slots of O are zeros
        // the log-sum-exp of a real query's logits: reference (mrun, natural units)
        // plus the log of the row sum
        if (lse != nullptr && r >= 0 && grp == 0)
            lse[(uint64_t)(uint32_t)r * (uint32_t)g.heads + h] = mrun + log2f(osum[0]) * kLn2;
        if (orow >= 0 && n < N) {
            const float inv = r >= 0 ? __builtin_amdgcn_rcpf(osum[0]) : 0.f;
            uint16_t* op = out + (uint64_t)(uint32_t)orow * (uint32_t)g.row + h * D + grp * 4;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const u32x2 w = {pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                 pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv)};
                *(u32x2*)(op + dt * 16) = w;
            }
        }
    }
}

// With 32-wide heads a workgroup's LDS is about half a CU's, so the 9-tile
// variant is held to 80 VGPRs: two workgroups of 12 waves then share a CU, and
// one computes while the other waits at its barriers.
template <int D, int NWAVES, int NL, int KT_FIXED, bool BIAS_VEC>
__global__ __launch_bounds__((NWAVES + NL) * 64)
__attribute__((amdgpu_waves_per_eu(D == 32 && BIAS_VEC && KT_FIXED == 9 && NWAVES + NL == 12 ? 6 : 1))) void
attn_bf16_stream_kernel(
    Geometry g, int staged, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ table, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int THREADS = (NWAVES + NL) * 64;
    static_assert(KT_FIXED <= NWAVES, "one query tile per compute wave");
    extern __shared__ __align__(16) unsigned char smem[];
    const StreamLds L = stream_lds(g);
    float* bias_lds = (float*)(smem + L.bias);
    int* kb4 = (int*)(smem + L.kb4);
    const int N = g.N, NP = L.NP;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const uint32_t units = (uint32_t)(g.windows * g.heads);
    const uint32_t per = gridDim.x / kXcds;
    const uint32_t xcd = blockIdx.x % kXcds;
    const uint32_t ubeg = (uint32_t)((uint64_t)units * xcd / kXcds);
    const uint32_t uend = (uint32_t)((uint64_t)units * (xcd + 1) / kXcds);
    const uint32_t u0 = ubeg + blockIdx.x / kXcds;
    if (u0 >= uend) return;

    // ---- window-independent tables (every head's bias, when resident, is the
    // compute waves' part of the prologue: below)
    for (int n = tid; n < NP; n += THREADS) {
        if (n < N) {
            int lt, ly, lx;
            local_coords(g, n, lt, ly, lx);
            kb4[n] = ((lt * g.tdy + ly) * g.tdx + lx) * 4;
        } else {
            kb4[n] = BIAS_VEC ? 12 : 0; // keeps qb - kb (- 3) inside the table
        }
    }

    if (wave >= NWAVES) {
        // ---- loader waves.  Token tables are built three units ahead and the
        // source offsets of each batch of copies while the previous batch is
        // awaited, so that after a barrier a loader only issues copies.
        constexpr int MAXC = loader_max_copies<D, KT_FIXED, NL>();
        constexpr int NCOPY = KT_FIXED * 16 * (D / 8) / 64; // copies per tensor (fixed tile counts)
        constexpr bool EX = KT_FIXED > 0 && NCOPY % NL == 0;
        const int j = wave - NWAVES;
        const LoaderRange R = loader_range(g, L, j, NL);
        // copies with a unit's K and Q, with its V, and O stores (one per 1 KB of rows)
        const int nkq = loader_kq_copies(g, L, j, NL), nv = loader_v_copies(g, L, j, NL), nst = nv;
        auto head = [&](uint32_t uu) { return (int)(uu - fdiv(g.fd_heads, uu) * (uint32_t)g.heads); };
        uint32_t okq[MAXC], ov[MAXC]; // source offsets of the next K/Q and V copies
        const uint32_t u1 = u0 + per, u2 = u1 + per;
        stream_table<D>(g, L, smem, R, lane, u0, 0, staged);
        stream_offsets<D, MAXC, EX>(g, L, smem, R, lane, 0, okq);
        stream_copy_kq<D, MAXC, EX>(g, L, smem, j, R, lane, head(u0), okq, 0, 0, q, k, table);
        stream_offsets<D, MAXC, EX>(g, L, smem, R, lane, 0, ov);
        stream_issue<D, MAXC, EX>(R, head(u0), ov, v, smem + L.v0);
        if (u1 < uend) {
            stream_table<D>(g, L, smem, R, lane, u1, 1, staged);
            stream_offsets<D, MAXC, EX>(g, L, smem, R, lane, 1, okq);
            stream_copy_kq<D, MAXC, EX>(g, L, smem, j, R, lane, head(u1), okq, 1, 1, q, k, table);
            stream_offsets<D, MAXC, EX>(g, L, smem, R, lane, 1, ov);
        }
        if (u2 < uend) stream_table<D>(g, L, smem, R, lane, u2, 2, staged);
        loader_barrier(); // prologue: window-independent tables and the first token tables
        // Issue order (loader j): K0 Q0 V0 K1 Q1 | after A_i: V(i+1), O(i-1) stores |
        // after B_i: K(i+2) Q(i+2).  Vector memory operations of a wave complete in
        // order, so each wait counts what was issued after the awaited copies.
        uint32_t u = u0;
        for (int iter = 0;; iter++) {
            const uint32_t un = u + per, un2 = un + per, un3 = un2 + per;
            const bool has_next = un < uend;
            // A: K, Q of unit u have landed once at most V(u), O(u-2) stores and
            // K/Q(un) remain
            wait_vmcnt_le(nv + (iter >= 2 ? nst : 0) + (has_next ? nkq : 0));
            loader_barrier();
            if (has_next) stream_issue<D, MAXC, EX>(R, head(un), ov, v, smem + L.v0 + ((iter + 1) % kBufs) * L.tb);
            if (iter >= 1) // O of the previous unit, staged by the compute waves before A
                stream_store_o<D, MAXC, EX>(g, L, smem, out, R, lane, u - per, (iter - 1) % kTableSlots, staged);
            if (un2 < uend) stream_offsets<D, MAXC, EX>(g, L, smem, R, lane, (iter + 2) % kTableSlots, okq);
            // B: V of unit u has landed once at most O(u-2) stores, K/Q(un), V(un)
            // and O(u-1) stores remain
            wait_vmcnt_le((iter >= 2 ? nst : 0) + (has_next ? nkq + nv : 0) + (iter >= 1 ? nst : 0));
            loader_barrier();
            if (un2 < uend) {
                stream_copy_kq<D, MAXC, EX>(g, L, smem, j, R, lane, head(un2), okq, (iter + 2) % kTableSlots, iter % kBufs,
                                        q, k, table);
                stream_offsets<D, MAXC, EX>(g, L, smem, R, lane, (iter + 2) % kTableSlots, ov);
            }
            if (un3 < uend) stream_table<D>(g, L, smem, R, lane, un3, (iter + 3) % kTableSlots, staged);
            if (!has_next) break;
            u = un;
        }
        // O of the last unit, staged before the final barrier
        loader_barrier();
        stream_store_o<D, MAXC, EX>(g, L, smem, out, R, lane, u, (int)((uend - 1 - u0) / per) % kTableSlots, staged);
    } else {
        // ---- compute waves.  Every head's bias slice when resident, from the
        // table read in its own order (coalesced), while the loaders already
        // build the first units' tables and issue their copies.
        if (L.bias_resident) {
            const uint32_t n = (uint32_t)g.table_size * (uint32_t)g.heads;
            for (uint32_t e = (uint32_t)tid; e < n; e += NWAVES * 64) {
                const uint32_t i = fdiv(g.fd_heads, e);
                bias_lds[(e - i * (uint32_t)g.heads) * L.TSP + i] = table[e];
            }
        }
        const int KT = KT_FIXED > 0 ? KT_FIXED : NP / 16;
        const bool active = wave < KT;
        TileState<(KT_FIXED > 0 ? KT_FIXED : kStreamMaxTiles)> ts;
        BiasOffsets<KT_FIXED, BIAS_VEC> bo;
        lds_barrier(); // prologue
        if (active) bias_offsets<KT_FIXED, BIAS_VEC>(g, L, smem, wave, lane, bo);
        uint32_t u = u0;
        for (int iter = 0;; iter++) {
            const int s = iter % kTableSlots, b = iter % kBufs;
            lds_barrier(); // A
            if (active) stream_qk<D, KT_FIXED, BIAS_VEC>(g, L, smem, wave, lane, u, s, b, bo, ts);
            lds_barrier(); // B
            if (active)
                stream_pv<D, KT_FIXED>(L, smem, lane, b, ts, lse, (int)(u - fdiv(g.fd_heads, u) * (uint32_t)g.heads),
                                       g.heads);
            u += per;
            if (u >= uend) break;
        }
        lds_barrier(); // final: the last O tile is staged
    }
}

// bf16 attention kernels share one signature: (geometry, staged, q, k, v, table, out)
typedef void (*bf16_kernel_t)(Geometry, int, const uint16_t*, const uint16_t*, const uint16_t*,
                              const float*, uint16_t*, float*);

// --------------------------------------------------------------------------
// bf16 attention, key-blocked schedule: windows whose K and V do not fit in
// one workgroup's LDS, e.g. the 32 x 32 windows (N = 1024) of TERRA's Large
// model (TERRA page, Table V).  There the path turns MFMA-bound: the
// intensity is N / 2 FLOP per byte, 512 against a ridge near 315.
//
// A workgroup takes kKbQueries queries of one (window, head).  Each of its
// eight compute waves holds two 16-query tiles of Q in registers, so every K
// and V fragment it reads from LDS feeds two MFMAs.  Two loader waves stream
// K and V in blocks of 32 keys through a ring of LDS stages with
// global_load_lds (the swizzled [key][d] layout of the other bf16 kernels)
// and the compute waves run an online softmax over the blocks.  The logits
// come straight out of the MFMA: its accumulator starts at bias / scale, so
// S^T holds q.k + bias / scale and the exponent is one FMA with scale *
// log2(e).  The exponent's reference M per query moves lazily: a block
// whose logits all stay within 2^8 of exp2(M) (a per-lane test and one
// ballot) is exponentiated against M as it stands (P <= 256, exact in the
// final ratio, and fp32 sums cannot overflow); otherwise the wave takes the
// exact block max across lanes, M moves to it and O and the row sum are
// rescaled.  Softmax is invariant to the reference, so the result is the
// same function; only rounding differs.  One barrier per
// block: at barrier j block j has landed and block j - 1 is no longer read,
// so the loaders refill its stage with block j + stages - 1; a wave's vector
// memory operations complete in order, so the loaders' waits are exact
// counts.  The head's bias slice is read from a head-major copy of the table
// holding bias / scale (one contiguous read instead of one line per entry,
// refreshed by a small kernel before each launch).  At the end the
// compute waves stage their O rows in the ring and store whole token rows.
// --------------------------------------------------------------------------
constexpr int kKbWaveQueries = 32;
constexpr int kKbComputeWaves = 8;
constexpr int kKbLoaders = 2;
constexpr int kKbQueries = kKbWaveQueries * kKbComputeWaves; // per workgroup
constexpr int kKbKeys = 32;                                   // keys per block
constexpr int kKbMaxStages = 8;
constexpr int kKbMinStages = 3;
constexpr float kKbSlack = 8.f; // log2 of the largest P before the reference max moves

struct KbLds {
    int NK, NT, stages; // keys rounded up to whole blocks; table words; ring stages
    size_t stage_bytes, ring_bytes, bias, tw, kb4, total;
};

__host__ __device__ inline KbLds kb_lds(const Geometry& g) {
    KbLds L;
    L.NK = (g.N + kKbKeys - 1) / kKbKeys * kKbKeys;
    const int NQ = (g.N + kKbQueries - 1) / kKbQueries * kKbQueries;
    L.NT = L.NK > NQ ? L.NK : NQ;
    L.stage_bytes = (size_t)2 * kKbKeys * g.head_dim * 2; // K, then V
    const size_t bias_bytes = ((size_t)g.table_size * 4 + 15) / 16 * 16;
    const size_t fixed = bias_bytes + (size_t)L.NT * 4 + (size_t)L.NK * 4;
    const size_t staging = (size_t)kKbQueries * g.head_dim * 2; // O rows, at the end
    int st = kKbMaxStages;
    while (st > 1 && fixed + (size_t)st * L.stage_bytes > (size_t)kLdsBytes) st--;
    L.stages = st;
    L.ring_bytes = (size_t)st * L.stage_bytes > staging ? (size_t)st * L.stage_bytes : staging;
    L.bias = L.ring_bytes;
    L.tw = L.bias + bias_bytes;
    L.kb4 = L.tw + (size_t)L.NT * 4;
    L.total = L.kb4 + (size_t)L.NK * 4;
    return L;
}

// dst[h][i] = table[i][h] / scale (scale 1: an exact copy)
__global__ __launch_bounds__(256) void bias_head_major_kernel(int table_size, int heads, float scale,
                                                              const float* __restrict__ table,
                                                              float* __restrict__ dst) {
    const int64_t n = (int64_t)table_size * heads;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / heads;
        const int hh = (int)(e - i * heads);
        dst[(int64_t)hh * table_size + i] = table[e] / scale;
    }
}

template <int D, bool BIAS_VEC>
__global__ __launch_bounds__((kKbComputeWaves + kKbLoaders) * 64) void attn_bf16_kblock_kernel(
    Geometry g, int staged, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ bias_hm, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int THREADS = (kKbComputeWaves + kKbLoaders) * 64;
    constexpr int KSTEPS = D / 32, DT = D / 16, CH = D / 8, RPC = 64 / CH;
    constexpr int KCOPIES = kKbKeys * CH / 64;        // 1 KB copies per tensor per block
    constexpr int LCOPIES = 2 * KCOPIES / kKbLoaders; // per loader wave per block
    static_assert((2 * KCOPIES) % kKbLoaders == 0, "the copies of a block divide among the loaders");
    extern __shared__ __align__(16) unsigned char smem[];
    const KbLds L = kb_lds(g);
    float* bias = (float*)(smem + L.bias);
    int* tw = (int*)(smem + L.tw);
    int* kb4 = (int*)(smem + L.kb4);
    const int N = g.N;
    const int NB = L.NK / kKbKeys, S = L.stages;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int nqb = (N + kKbQueries - 1) / kKbQueries;

    // block -> (window, head, query block): the query blocks and heads of a
    // window run side by side on one XCD and share its L2 copy of K and V
    const int64_t work = xcd_work_index(blockIdx.x, g.windows * g.heads * nqb);
    const int64_t wh = work / nqb;
    const int qblk = (int)(work - wh * nqb);
    const uint32_t wi = (uint32_t)(wh / g.heads);
    const int h = (int)(wh - (int64_t)wi * g.heads);
    const int b = (int)fdiv(g.fd_nW, wi);
    int wc[3];
    {
        const uint32_t r = wi - (uint32_t)b * (uint32_t)g.nW;
        const uint32_t r2 = fdiv(g.fd_nwin2, r);
        wc[2] = (int)(r - r2 * (uint32_t)g.nwin[2]);
        wc[0] = (int)fdiv(g.fd_nwin1, r2);
        wc[1] = (int)(r2 - (uint32_t)wc[0] * (uint32_t)g.nwin[1]);
    }
    const bool masked_window = window_maybe_masked(g, wc);

    // ---- token table (packed as in the other bf16 kernels), key bias offsets
    // and this head's bias slice
    for (int n = tid; n < L.NT; n += THREADS) {
        if (n < N) {
            int l[3];
            local_coords(g, n, l[0], l[1], l[2]);
            int region = 0, tok = b;
            bool is_pad = false;
#pragma unroll
            for (int a = 0; a < 3; a++) {
                const int cr = wc[a] * g.win[a] + l[a];
                int c = cr + g.shift[a];
                if (c >= g.pad[a]) c -= g.pad[a];
                is_pad |= c >= g.ext[a];
                if (!g.cyc[a] && cr >= g.pad[a] - g.shift[a]) region |= 1 << a;
                tok = tok * g.ext[a] + c;
            }
            const int row = is_pad ? -1 : (staged ? (int)(wi * (uint32_t)N + n) : tok);
            tw[n] = (row + 1) | ((region | (is_pad ? 8 : 0)) << 28);
            if (n < L.NK) kb4[n] = ((l[0] * g.tdy + l[1]) * g.tdx + l[2]) * 4;
        } else {
            tw[n] = 15 << 28;
            if (n < L.NK) kb4[n] = BIAS_VEC ? 12 : 0; // keeps qb - kb (- 3) inside the table
        }
    }
    {
        const float* bsrc = bias_hm + (size_t)h * g.table_size;
        for (int i = tid; i < g.table_size; i += THREADS) bias[i] = bsrc[i];
    }
    __syncthreads();

    if (wave >= kKbComputeWaves) {
        // ---- loader waves: copies j * LCOPIES .. of every block (K copies, then V)
        const int j = wave - kKbComputeWaves;
        auto issue = [&](int blk) __attribute__((always_inline)) {
            unsigned char* st = smem + (size_t)(blk % S) * L.stage_bytes;
#pragma unroll
            for (int i = 0; i < LCOPIES; i++) {
                const int c = j * LCOPIES + i;
                const bool is_v = c >= KCOPIES;
                const int cc = is_v ? c - KCOPIES : c;
                const int m = cc * RPC + lane / CH; // key row in the block
                const int r1 = tw[blk * kKbKeys + m] & kRowMask;
                const uint64_t off = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + h * D +
                                     copy_chunk<D>(m, lane) * 8;
                __builtin_amdgcn_global_load_lds((const void*)((is_v ? v : k) + off),
                                                 (lds_void*)(st + (is_v ? kKbKeys * D * 2 : 0) + cc * 1024), 16, 0,
                                                 0);
            }
        };
        const int pre = NB < S - 1 ? NB : S - 1;
        for (int blk = 0; blk < pre; blk++) issue(blk);
        for (int blk = 0; blk < NB; blk++) {
            // block blk has landed once at most the blocks issued after it remain
            const int after = NB - 1 - blk < S - 2 ? NB - 1 - blk : S - 2;
            wait_vmcnt_le(after * LCOPIES);
            loader_barrier();
            if (blk + S - 1 < NB) issue(blk + S - 1);
        }
        loader_barrier(); // final: the ring is free for the O rows
        return;
    }

    // ---- compute waves: queries qbase .. qbase + 31 in two tiles
    const int qbase = qblk * kKbQueries + wave * kKbWaveQueries;
    const bool active = qbase < N;
    const unsigned one2 = 0x3F803F80u; // two bf16 ones
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});
    int qreg[2], qr[2], qb4[2];
    bf16x8 qf[2][KSTEPS]; // B operand: query n, d = 32 ks + 8 grp + 0..7
    f32x4 o[2][DT], osum[2];
    float mref[2];                       // exponent reference per query, log2 units
    const float c2 = g.scale * kLog2e;   // logits (q.k + bias / scale) to log2 units
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const int n = qbase + t * 16 + col;
        const int word = tw[n];
        qreg[t] = (unsigned)word >> 28;
        qr[t] = (word & kRowMask) - 1;
        if (n < N) {
            int lt, ly, lx;
            local_coords(g, n, lt, ly, lx);
            qb4[t] = (((lt * g.tdy + ly) * g.tdx + lx) + g.c0) * 4;
        } else {
            qb4[t] = (g.table_size - 1) * 4; // largest qb keeps qb - kb inside the table
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            u32x4 val = {0, 0, 0, 0};
            if (active && qr[t] >= 0)
                val = *(const u32x4*)(q + (uint64_t)(uint32_t)qr[t] * (uint32_t)g.row + h * D + ks * 32 + grp * 8);
            qf[t][ks] = __builtin_bit_cast(bf16x8, val);
        }
#pragma unroll
        for (int dt = 0; dt < DT; dt++) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        osum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        mref[t] = -INFINITY;
    }
    // A block that shares no mask field with any of the wave's 32 queries adds
    // P = 0 and leaves the exponent reference alone, so the wave skips it; a
    // wave of pad queries only (no output) skips every block.  A 32-key block
    // is one row of a 32-wide window, so where a window is split by the
    // non-cyclic boundary, each side's waves skip the other side's rows.
    unsigned qset = (1u << qreg[0]) | (1u << qreg[1]);
#pragma unroll
    for (int sh = 8; sh >= 1; sh >>= 1) qset |= __shfl_xor(qset, sh);
    qset = __builtin_amdgcn_readfirstlane(qset);
    const bool any_real = __builtin_amdgcn_ballot_w64(qr[0] >= 0 || qr[1] >= 0) != 0;

    for (int blk = 0; blk < NB; blk++) {
        lds_barrier();
        if (!active || !any_real) continue;
        if (masked_window) { // the fields present among the block's 32 keys
            const u32x4 f = *(const u32x4*)(tw + blk * kKbKeys + (lane & 7) * 4);
            unsigned m = (1u << (f[0] >> 28)) | (1u << (f[1] >> 28)) | (1u << (f[2] >> 28)) | (1u << (f[3] >> 28));
#pragma unroll
            for (int sh = 4; sh >= 1; sh >>= 1) m |= __shfl_xor(m, sh);
            if ((__builtin_amdgcn_readfirstlane(m) & qset) == 0) continue;
        }
        const unsigned char* st = smem + (size_t)(blk % S) * L.stage_bytes;
        const uint16_t* Ks = (const uint16_t*)st;
        const unsigned char* Vb = st + kKbKeys * D * 2;
        const int key_base = blk * kKbKeys;
        // S^T = K Q^T + bias / scale for both query tiles (the accumulators start at
        // the biases), each K fragment read once
        f32x4 sc[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            const int kq = key_base + kt * 16 + grp * 4;
            f32x4 acc[2];
            if (BIAS_VEC) {
                const int kb0 = kb4[kq]; // keys kq + i share a window row: biases at qb - kb0 - i
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const float* bp = (const float*)((const unsigned char*)bias + qb4[t] - kb0 - 12);
                    acc[t] = f32x4{bp[3], bp[2], bp[1], bp[0]};
                }
            } else {
                const int4 k4 = *(const int4*)(kb4 + kq);
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const unsigned char* qb = (const unsigned char*)bias + qb4[t];
                    acc[t] = f32x4{*(const float*)(qb - k4.x), *(const float*)(qb - k4.y),
                                   *(const float*)(qb - k4.z), *(const float*)(qb - k4.w)};
                }
            }
            const int krow = kt * 16 + col;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) {
                const bf16x8 a =
                    __builtin_bit_cast(bf16x8, *(const u32x4*)(Ks + krow * D + k_slot<D>(krow, ks * 4 + grp) * 8));
                acc[0] = mfma32(a, qf[0][ks], acc[0]);
                acc[1] = mfma32(a, qf[1][ks], acc[1]);
            }
            sc[0][kt] = acc[0];
            sc[1][kt] = acc[1];
        }
        // the mask, where keys can be hidden
        if (masked_window || key_base + kKbKeys > N) {
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
                const int4 kr4 = *(const int4*)(tw + key_base + kt * 16 + grp * 4);
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const unsigned qg = (unsigned)qreg[t];
                    sc[t][kt][0] = ((unsigned)kr4.x >> 28) == qg ? sc[t][kt][0] : -INFINITY;
                    sc[t][kt][1] = ((unsigned)kr4.y >> 28) == qg ? sc[t][kt][1] : -INFINITY;
                    sc[t][kt][2] = ((unsigned)kr4.z >> 28) == qg ? sc[t][kt][2] : -INFINITY;
                    sc[t][kt][3] = ((unsigned)kr4.w >> 28) == qg ? sc[t][kt][3] : -INFINITY;
                }
            }
        }
        // exponent reference: moves only when a logit passes it by more than the slack
        float lmax[2];
        bool grow = false;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            lmax[t] = fmaxf(fmaxf(fmaxf(sc[t][0][0], sc[t][0][1]), fmaxf(sc[t][0][2], sc[t][0][3])),
                            fmaxf(fmaxf(sc[t][1][0], sc[t][1][1]), fmaxf(sc[t][1][2], sc[t][1][3]))) * c2;
            grow |= lmax[t] > mref[t] + kKbSlack;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int t = 0; t < 2; t++) {
                float bm = fmaxf(lmax[t], __shfl_xor(lmax[t], 16));
                bm = fmaxf(bm, __shfl_xor(bm, 32));
                const float mn = fmaxf(mref[t], bm);
                const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref[t] - mn);
                osum[t] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; dt++) o[t][dt] *= alpha;
                mref[t] = mn;
            }
        }
        // P = exp2(c2 * logit - M), packed to bf16 (keys 0..31 of the block)
        bf16x8 bop[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const float mc = mref[t] == -INFINITY ? 0.f : mref[t];
            unsigned pk[4];
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[t][kt][i], c2, -mc));
                pk[2 * kt] = pack_bf16x2(p[0], p[1]);
                pk[2 * kt + 1] = pack_bf16x2(p[2], p[3]);
            }
            bop[t] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        }
        // O^T += V^T P^T, each V^T fragment read once for both tiles; the row sums with A = 1
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            u32x2 half[2];
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
                const int row = kt * 16 + grp * 4 + (col >> 2);
                const int d = dt * 16 + (col & 3) * 4;
                const unsigned char* p = Vb + row * (D * 2) + k_slot<D>(row, d >> 3) * 16 + (d & 7) * 2;
                half[kt] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_void*)p));
            }
            const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{half[0][0], half[0][1], half[1][0], half[1][1]});
            o[0][dt] = mfma32(a, bop[0], o[0][dt]);
            o[1][dt] = mfma32(a, bop[1], o[1][dt]);
        }
        osum[0] = mfma32(ones8, bop[0], osum[0]);
        osum[1] = mfma32(ones8, bop[1], osum[1]);
    }
    lds_barrier(); // final: every wave is done with the ring
    if (!active) return;

    // ---- O: divide by the sum, stage this wave's 32 rows in the ring, store whole rows
    uint16_t* Os = (uint16_t*)(smem + (size_t)wave * kKbWaveQueries * D * 2);
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const float inv = qr[t] >= 0 ? __builtin_amdgcn_rcpf(osum[t][0]) : 0.f;
        // the log-sum-exp of a real query's logits: reference (log2 units) plus the
        // log of the row sum
        if (lse != nullptr && qr[t] >= 0 && grp == 0)
            lse[(uint64_t)(uint32_t)qr[t] * (uint32_t)g.heads + h] = (mref[t] + log2f(osum[t][0])) * kLn2;
        const int m = t * 16 + col;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const u32x2 w = {pack_bf16x2(o[t][dt][0] * inv, o[t][dt][1] * inv),
                             pack_bf16x2(o[t][dt][2] * inv, o[t][dt][3] * inv)};
            const int c = dt * 2 + (grp >> 1); // 16-byte chunk of d = 16 dt + 4 grp
            *(u32x2*)(Os + m * D + k_slot<D>(m, c) * 8 + (grp & 1) * 4) = w;
        }
    }
#pragma unroll
    for (int i = 0; i < kKbWaveQueries / RPC; i++) {
        const int m = i * RPC + lane / CH, c = lane % CH;
        const u32x4 val = *(const u32x4*)(Os + m * D + k_slot<D>(m, c) * 8);
        const int n = qbase + m;
        const int r = (tw[n] & kRowMask) - 1;
        // staged: pad slots of the window-major output get zeros (their sums are 0)
        const int64_t orow = r >= 0 ? (int64_t)r : (staged && n < N ? (int64_t)wi * N + n : -1);
        if (orow >= 0)
            __builtin_nontemporal_store(val, (u32x4*)(out + orow * g.row + h * D + c * 8));
    }
}

bool bf16_kblock_fits(const Geometry& g) {
    const KbLds L = kb_lds(g);
    const int64_t rows = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    const int64_t wrows = g.windows * g.N;
    return L.total <= (size_t)kLdsBytes && L.stages >= kKbMinStages && (rows > wrows ? rows : wrows) < kRowMask &&
           g.windows * g.heads * ((g.N + kKbQueries - 1) / kKbQueries) < ((int64_t)1 << 31);
}

size_t bf16_kblock_workspace_bytes(const Geometry& g) { return (size_t)g.table_size * g.heads * sizeof(float); }

template <int D>
static bf16_kernel_t kblock_variant(bool bv) {
    return bv ? attn_bf16_kblock_kernel<D, true> : attn_bf16_kblock_kernel<D, false>;
}

static bf16_kernel_t kblock_variant_for(const Geometry& g) {
    const bool bv = g.win[2] % 4 == 0;
    if (g.head_dim == 32) return kblock_variant<32>(bv);
    if (g.head_dim == 128) return kblock_variant<128>(bv);
    return kblock_variant<64>(bv);
}

static int64_t kblock_workgroups(const Geometry& g) {
    return g.windows * g.heads * ((g.N + kKbQueries - 1) / kKbQueries);
}

hipError_t kblock_plan(const Geometry& g, int* blocks) {
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, (const void*)kblock_variant_for(g), (kKbComputeWaves + kKbLoaders) * 64, kb_lds(g).total);
    if (e != hipSuccess) return e;
    *blocks = per_cu < 1 ? 0 : (int)kblock_workgroups(g);
    return hipSuccess;
}

hipError_t launch_attention_kblock(const Geometry& g, bool staged, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const float* table, float* bias_hm, uint16_t* out,
                                   float* lse, hipStream_t s) {
    const int64_t n = (int64_t)g.table_size * g.heads;
    const int64_t tb = (n + 255) / 256;
    hipLaunchKernelGGL(bias_head_major_kernel, dim3((unsigned)(tb < 1024 ? tb : 1024)), dim3(256), 0, s,
                       g.table_size, g.heads, g.scale, table, bias_hm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kblock_variant_for(g), dim3((unsigned)kblock_workgroups(g)),
                       dim3((kKbComputeWaves + kKbLoaders) * 64), kb_lds(g).total, s, g, (int)staged, q, k, v,
                       (const float*)bias_hm, out, lse);
    return hipGetLastError();
}

size_t attention_lds_bytes(const Geometry& g, bool bf16, bool staged) {
    if (!bf16) return f32_lds_bytes(g);
    // the smallest footprint among the bf16 schedules that can take the window
    size_t best = (size_t)-1;
    if (bf16_stream_fits(g, staged)) best = stream_lds(g).total;
    if (bf16_block_fits(g) && bf16_lds(g).total < best) best = bf16_lds(g).total;
    if (bf16_kblock_fits(g) && kb_lds(g).total < best) best = kb_lds(g).total;
    return best;
}

// Kernel variant for a geometry: specialised tile counts, else the general one.
struct Bf16Variant {
    bf16_kernel_t f;
    int waves; // waves per workgroup
};

template <int D, bool BV>
static Bf16Variant bf16_variant_b(int KT) {
    if constexpr (D == 128) { // 128-wide heads: the general tile counts only
        if (KT <= 8) return {attn_bf16_kernel<D, 8, 1, 0, BV>, 8};
        return {attn_bf16_kernel<D, 8, 4, 0, BV>, 8};
    } else {
        switch (KT) {
        case 4: return {attn_bf16_kernel<D, 4, 1, 4, BV>, 4};
        case 7: return {attn_bf16_kernel<D, 7, 1, 7, BV>, 7};
        case 9: return {attn_bf16_kernel<D, 9, 1, 9, BV>, 9};
        // 18 tiles (e.g. 2 x 12 x 12 windows): 8 waves of up to 3 tiles, so that two
        // workgroups (80 KB of LDS each, 4 waves per SIMD) share a compute unit
        case 18: return {attn_bf16_kernel<D, 8, 3, 18, BV>, 8};
        default:
            if (KT <= 8) return {attn_bf16_kernel<D, 8, 1, 0, BV>, 8};
            return {attn_bf16_kernel<D, 8, 4, 0, BV>, 8};
        }
    }
}

// Loader waves of a streaming variant.  Issuing the copies is what limits a
// loader wave, so the 64-wide variants take as many as their registers allow
// (15 or 16 waves per workgroup, four per SIMD) and divide the copies evenly
// (18 or 14 per tensor); the 128-wide 4-tile variant takes four (16 copies per
// tensor); the others take three.
template <int D, int KT, bool BV>
constexpr int stream_loaders() {
    return D == 64 && KT == 7 ? 7 : (D == 64 && KT == 9 && BV ? 6 : (D == 128 && KT == 4 ? 4 : 3));
}

template <int D, int NWAVES, int KT, bool BV>
static Bf16Variant stream_variant() {
    constexpr int NL = stream_loaders<D, KT, BV>();
    return {attn_bf16_stream_kernel<D, NWAVES, NL, KT, BV>, NWAVES + NL};
}

template <int D, bool BV>
static Bf16Variant stream_variant_b(int KT) {
    if constexpr (D == 128) { // 128-wide heads: LDS holds the buffers of windows of up to 5 tiles
        if (KT == 4) return stream_variant<D, 4, 4, BV>();
        return stream_variant<D, kStreamMaxTiles128, 0, BV>();
    } else {
        switch (KT) {
        case 4: return stream_variant<D, 4, 4, BV>();
        case 7: return stream_variant<D, 7, 7, BV>();
        case 9: return stream_variant<D, 9, 9, BV>();
        default: return stream_variant<D, kStreamMaxTiles, 0, BV>();
        }
    }
}

static Bf16Variant bf16_variant_for(const Geometry& g, bool stream) {
    const int KT = (g.N + 15) / 16;
    const bool bv = g.win[2] % 4 == 0;
    if (stream) {
        if (g.head_dim == 32) return bv ? stream_variant_b<32, true>(KT) : stream_variant_b<32, false>(KT);
        if (g.head_dim == 128) return bv ? stream_variant_b<128, true>(KT) : stream_variant_b<128, false>(KT);
        return bv ? stream_variant_b<64, true>(KT) : stream_variant_b<64, false>(KT);
    }
    if (g.head_dim == 32) return bv ? bf16_variant_b<32, true>(KT) : bf16_variant_b<32, false>(KT);
    if (g.head_dim == 128) return bv ? bf16_variant_b<128, true>(KT) : bf16_variant_b<128, false>(KT);
    return bv ? bf16_variant_b<64, true>(KT) : bf16_variant_b<64, false>(KT);
}

bool bf16_block_fits(const Geometry& g) {
    const int64_t rows = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    const int64_t wrows = g.windows * g.N;
    // the general per-unit variant takes up to 8 waves x 4 tiles = 512 tokens; row + 1
    // of the real-token layout (fused) or of the window slots (staged) fits the 28 bits
    // of the packed table word
    return g.N <= 512 && bf16_lds(g).total <= (size_t)kLdsBytes && (rows > wrows ? rows : wrows) < kRowMask;
}

bool bf16_stream_fits(const Geometry& g, bool staged) {
    // the layout the kernel reads and writes: real tokens (fused) or window slots (staged)
    const int64_t rows = staged ? g.windows * g.N : (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    const int KT = (g.N + 15) / 16;
    // row + 1 fits the packed table word; the loaders' element offsets fit 32 bits; the
    // O stores' buffer offsets, from the start of the unit's batch item, stay below 2^31
    return stream_lds(g).total <= (size_t)kLdsBytes && KT <= (g.head_dim == 128 ? kStreamMaxTiles128 : kStreamMaxTiles) &&
           rows < kRowMask && (uint64_t)rows * (uint64_t)g.row < ((uint64_t)1 << 32) &&
           stream_item_bytes(g, staged) < kOutOfRange;
}

hipError_t bf16_plan(const Geometry& g, bool stream, int* blocks) {
    const Bf16Variant var = bf16_variant_for(g, stream);
    const size_t lds = stream ? stream_lds(g).total : bf16_lds(g).total;
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)var.f, var.waves * 64, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) {
        *blocks = 0;
        return hipSuccess;
    }
    if (!stream) {
        *blocks = (int)(g.windows * g.heads);
        return hipSuccess;
    }
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t n = (int64_t)per_cu * cus / kXcds * kXcds; // a multiple of the XCD count
    *blocks = (int)(n < kXcds ? kXcds : n);
    return hipSuccess;
}

hipError_t launch_attention_bf16(const Geometry& g, bool stream, int blocks, bool staged, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const float* table, float* bias_hm,
                                 uint16_t* out, float* lse, hipStream_t s) {
    const Bf16Variant var = bf16_variant_for(g, stream);
    const size_t lds = stream ? stream_lds(g).total : bf16_lds(g).total;
    if (!stream) { // the per-unit kernel reads its head's bias slice from a head-major copy
        const int64_t n = (int64_t)g.table_size * g.heads;
        const int64_t tb = (n + 255) / 256;
        hipLaunchKernelGGL(bias_head_major_kernel, dim3((unsigned)(tb < 1024 ? tb : 1024)), dim3(256), 0, s,
                           g.table_size, g.heads, 1.0f, table, bias_hm);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        table = bias_hm;
    }
    hipLaunchKernelGGL(var.f, dim3((unsigned)blocks), dim3(var.waves * 64), lds, s, g,
                       (int)staged, q, k, v, table, out, lse);
    return hipGetLastError();
}

hipError_t prepare_kernels(int max_lds) {
    const void* f32k[] = {(const void*)attn_f32_kernel<32>, (const void*)attn_f32_kernel<64>};
    for (const void* f : f32k) {
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
        if (e != hipSuccess) return e;
    }
    for (int stream = 0; stream < 2; stream++) {
        for (int KT : {4, 7, 9, 18, 1, 32}) {
            const bf16_kernel_t fs[] = {
                stream ? stream_variant_b<32, true>(KT).f : bf16_variant_b<32, true>(KT).f,
                stream ? stream_variant_b<32, false>(KT).f : bf16_variant_b<32, false>(KT).f,
                stream ? stream_variant_b<64, true>(KT).f : bf16_variant_b<64, true>(KT).f,
                stream ? stream_variant_b<64, false>(KT).f : bf16_variant_b<64, false>(KT).f,
                stream ? stream_variant_b<128, true>(KT).f : bf16_variant_b<128, true>(KT).f,
                stream ? stream_variant_b<128, false>(KT).f : bf16_variant_b<128, false>(KT).f};
            for (bf16_kernel_t f : fs) {
                hipError_t e =
                    hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
                if (e != hipSuccess) return e;
            }
        }
    }
    for (bool bv : {true, false}) {
        for (bf16_kernel_t f : {kblock_variant<32>(bv), kblock_variant<64>(bv), kblock_variant<128>(bv)}) {
            hipError_t e = hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

} // namespace swa
