// The window attention of a Swin block with its query/key/value projection
// fused in (TERRA page, abstract: the models are stacks of Swin blocks whose
// attention runs inside shifted windows; Table V: embedding width d = N_h
// heads x head_dim).  For every window, one workgroup computes, head by head,
//
//   q, k, v = x_w W_h^T + b_h       (x_w: the window's tokens, [N][C]; W_h: the
//                                    3 head_dim rows of W_qkv that head h owns)
//   o_h     = the window attention of that head on q, k, v
//
// and writes o_h to the attention-output tensor [token][heads][head_dim]; the
// output projection y = o W_o^T + b_o then runs as a separate GEMM.  So q, k
// and v never leave the chip: the token embeddings are read from HBM once
// (and from L2 for every further head), the weights from L2.  A workgroup
// takes a group of heads of one window (two when the head count is even);
// the groups of a window run side by side on one XCD and share its token rows
// in L2.
//
// A workgroup has 12 waves: 9 compute waves (one per query tile) for 9-tile
// windows of heads up to 64 wide, else 8, and the rest loader waves.  The
// loaders stream the reduction over the C input channels in stages of 64
// (whole 128-byte lines; 32 for 128-wide heads, for the LDS): a stage holds
// the window's token rows [NP][64] and the head's weight rows
// [3 head_dim][64] (bf16, 16-byte chunks XOR-swizzled by row), copied straight
// into an LDS ring of 2 to 4 slots, one fewer stages ahead, with
// global_load_lds; each loader's source offsets are computed once.  With a
// head's first stage they also copy its bias-table slice and its 3 head_dim
// projection biases into slots of that head's parity.  Pad tokens copy row 0
// (finite values whose keys are masked and whose outputs are dropped).
//
// Compute waves: wave (wf, wt) holds FTW feature tiles x up to TTW token tiles
// of the transposed product (features x tokens), 32-deep bf16 MFMA with fp32
// accumulation, in the same operand order and reduction order as the
// projection GEMM (swa_projection.hip); after a head's last stage each lane
// adds the fp32 biases and rounds once to bf16, writing its 4 features of one
// token into q, k or v ([token][head_dim], the streaming attention layout).
// So q, k, v equal the unfused projection's bit for bit.  Then each wave
// takes its query tile (and tile wave + 8 with 8 compute waves), one after the
// other: S^T = K Q^T,
// bias, mask and softmax (the streaming schedule's stream_qk), then O^T =
// V^T P^T written over the tile's own rows of Q (stream_pv; no other wave
// reads them), a barrier, and the compute waves store O's token rows
// (head_dim x 2 bytes each) with buffer stores, pad rows dropped by the range
// check.  The attention arithmetic is the streaming schedule's, instruction
// for instruction, so o equals swa_forward's on the same q, k, v bit for bit.
//
// Barriers: one per stage (the ring: a stage's copies have landed and the
// slot read the stage before is free), plus one per head (O is in LDS).
//
// What bounds it: every window re-streams its token rows once per head and
// every head's weights once per window, about 11 GB from L2 into LDS for the
// 540 x 1080 grid at C = 512, while the projection GEMM reads the tokens once
// per 256-feature tile; both the copies and the fragment reads of the small
// per-window products leave the matrix cores idle most of the time.  On the
// 540 x 1080, 180 x 360 and Table V Small shapes the unfused layer is faster,
// so AUTO takes it; the fused path needs a quarter of the workspace.  Loader and compute waves run separate loops
// with the same barrier count; the barriers fence LDS only.
#include "swa_device.h"
#include "swa_geometry.h"
#include "swa_layer.h"
#include "swa_stream.h"

namespace swa {
namespace {

constexpr int kLWaves = 12;  // waves per workgroup: compute waves, then loader waves
// Compute waves: one per query tile for 9-tile windows of heads up to 64 wide
// (3 x 3 groups of the projection), else 8 (3-tile feature groups).
template <int D, int KT>
constexpr int layer_compute_waves() { return KT == 9 && D <= 64 ? 9 : 8; }
// Input channels per stage: 64 (whole 128-byte lines of token and weight
// rows) for heads of up to 64, 32 for 128-wide heads, whose weight rows of a
// 64-channel stage would not fit the LDS next to q, k, v.  The ring holds
// layer_min_stages<SK>() stages (copied slots - 1 ahead), one more where it
// fits.
template <int D>
constexpr int layer_stage_channels() { return D == 128 ? 32 : 64; }
template <int SK>
constexpr int layer_min_stages() { return SK == 64 ? 2 : 3; }
#ifndef SWA_LAYER_HEADS
#define SWA_LAYER_HEADS 2 // heads per workgroup when the head count allows
#endif

struct LayerLds {
    int NP, TSP, F, BQP; // padded tokens; bias slice and projection-bias slot floats (multiples of 64); 3 head_dim
    size_t xst, stage;   // bytes of a stage's token rows; of a whole stage (tokens, then weights)
    size_t ring, q, k, v, tb, bias, bqkv, tw, kb4, total;
};

__host__ __device__ inline LayerLds layer_lds(const Geometry& g, int stages, int kLK) {
    LayerLds L;
    L.NP = (g.N + 15) / 16 * 16;
    L.TSP = (g.table_size + 63) / 64 * 64;
    L.F = 3 * g.head_dim;
    L.BQP = (L.F + 63) / 64 * 64;
    L.xst = (size_t)L.NP * kLK * 2;
    L.stage = L.xst + (size_t)L.F * kLK * 2;
    L.tb = (size_t)L.NP * g.head_dim * 2;
    L.ring = 0;
    L.q = L.ring + stages * L.stage;
    L.k = L.q + L.tb;
    L.v = L.k + L.tb;
    L.bias = L.v + L.tb;                       // two slots (head parity)
    L.bqkv = L.bias + 2 * (size_t)L.TSP * 4;  // two slots
    L.tw = L.bqkv + 2 * (size_t)L.BQP * 4;
    L.kb4 = L.tw + (size_t)L.NP * 4;
    L.total = L.kb4 + (size_t)L.NP * 4;
    return L;
}

// The streaming schedule's view of this LDS, for its query-tile halves: one
// buffer each of K, Q, V; O written over Q (a tile's O rows over its own Q
// rows); the bias slice in slot s = head parity; one token table (slot stride 0).
__device__ inline StreamLds stream_view(const LayerLds& F) {
    StreamLds L;
    L.NP = F.NP;
    L.TSP = F.TSP;
    L.bias_resident = false;
    L.tb = F.tb;
    L.k0 = F.k;
    L.q0 = F.q;
    L.v0 = F.v;
    L.o0 = F.q;
    L.bias = F.bias;
    L.kb4 = F.kb4;
    L.slot0 = F.tw;
    L.slot_bytes = 0;
    L.total = F.total;
    return L;
}

// Grid: one workgroup per (window, group of HG heads); the groups of a window
// are consecutive work items, so they run side by side on one XCD and read the
// window's token rows from its L2.
template <int D, int KT, bool BIAS_VEC, int NS>
__global__ __launch_bounds__(kLWaves * 64) void layer_qkv_attn_kernel(
    Geometry g, int HG, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bqkv,
    const float* __restrict__ table, uint16_t* __restrict__ o) {
    constexpr int THREADS = kLWaves * 64;
    constexpr int kLK = layer_stage_channels<D>();
    constexpr int kLC = layer_compute_waves<D, KT>();
    constexpr int kLL = kLWaves - kLC; // loader waves
    constexpr int F = 3 * D;      // projected features per head
    constexpr int FT = F / 16;    // feature tiles
    constexpr int WF = kLC == 9 ? 3 : FT / 3; // feature groups
    constexpr int FTW = FT / WF;  // feature tiles per wave
    constexpr int WT = kLC / WF;  // token groups
    static_assert(FTW * WF == FT && WF * WT == kLC, "feature and token groups over the compute waves");
    constexpr int TTW = (KT + WT - 1) / WT; // most token tiles of a wave
    constexpr int NP = KT * 16;
    constexpr int LPR = kLK * 2 / 16;   // lanes per row of a stage (16 bytes each)
    constexpr int RPC = 64 / LPR;       // rows per 1 KB copy
    constexpr int XC = NP / RPC;        // 1 KB copies of a stage's token rows
    constexpr int WC = F / RPC;         // of its weight rows
    constexpr int KSTEP = kLK / 32;     // 32-deep products per stage
    constexpr int QT = (KT + kLC - 1) / kLC; // query tiles per compute wave
    extern __shared__ __align__(16) unsigned char smem[];
    const LayerLds LL = layer_lds(g, NS, kLK);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = g.row;
    const int KS = C / kLK;          // stages per head
    const int steps = HG * KS;
    const uint32_t NG = (uint32_t)(g.heads / HG);
    const uint32_t item = (uint32_t)xcd_work_index(blockIdx.x, g.windows * NG);
    const uint32_t wi = item / NG;
    const int h0 = (int)(item - wi * NG) * HG; // first head of the group
    int* tw = (int*)(smem + LL.tw);
    int* kb4 = (int*)(smem + LL.kb4);

    // ---- the window's token table ((source row + 1) | mask field << 28, as the
    // streaming schedule builds it) and every key's bias offset
    {
        const Unit U = decode_unit(g, wi * (uint32_t)g.heads);
        for (int n = tid; n < NP; n += THREADS) {
            if (n < g.N) {
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
                tw[n] = (is_pad ? 0 : tok + 1) | ((region | (is_pad ? 8 : 0)) << 28);
                kb4[n] = ((l[0] * g.tdy + l[1]) * g.tdx + l[2]) * 4;
            } else {
                tw[n] = 15 << 28;
                kb4[n] = BIAS_VEC ? 12 : 0; // keeps qb - kb (- 3) inside the table
            }
        }
    }
    __syncthreads();

    if (wave >= kLC) {
        // ---- loader waves: copy c of a stage (tokens 0 .. XC-1, then weights) by
        // loader c % kLL; lane l lands 16 bytes in row 16 * copy + l / 4 at chunk
        // position l % 4, which holds logical chunk (l % 4) ^ ((row / 2) % 4)
        const int j = wave - kLC;
        // this loader's copies c = j, j + kLL, ... and their source offsets (in
        // elements, before the stage's channel offset and the head's weight rows):
        // computed once, so that issuing a stage reads no LDS
        constexpr int MAXC = (XC + WC + kLL - 1) / kLL;
        uint32_t off[MAXC];
        const int nc = (XC + WC - j + kLL - 1) / kLL;
#pragma unroll
        for (int i = 0; i < MAXC; i++) {
            const int c = j + i * kLL;
            const int cc = c < XC ? c : c - XC;
            const int r = cc * RPC + lane / LPR;
            const int ch = k_slot<kLK>(r, lane % LPR); // the logical chunk that lands in this lane's slot
            if (c < XC) {
                const int r1 = tw[r] & kRowMask;
                off[i] = (uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)C + ch * 8;
            } else {
                const int part = r / D, d = r - part * D; // feature r of the head: q, k or v row d
                off[i] = (uint32_t)(part * C + d) * (uint32_t)C + ch * 8;
            }
        }
        auto copies = [&](int s) __attribute__((always_inline)) {
            if (s >= steps) return 0;
            int n = nc;
            if (s % KS == 0) n += (LL.TSP / 64 - j + kLL - 1) / kLL + (LL.BQP / 64 - j + kLL - 1) / kLL;
            return n;
        };
        auto issue = [&](int s) __attribute__((always_inline)) {
            if (s >= steps) return;
            const int hl = s / KS, kc = s - hl * KS, h = h0 + hl;
            unsigned char* slot = smem + LL.ring + (s % NS) * LL.stage;
            const uint32_t wh = (uint32_t)(h * D) * (uint32_t)C; // head h's rows of each of q, k, v
#pragma unroll
            for (int i = 0; i < MAXC; i++) {
                if (i < nc) {
                    const int c = j + i * kLL;
                    const bool tok = c < XC;
                    const uint16_t* src = tok ? x + off[i] + kc * kLK : w + (off[i] + wh) + kc * kLK;
                    __builtin_amdgcn_global_load_lds((const void*)src,
                                                     (lds_void*)(slot + (tok ? c * 1024 : LL.xst + (c - XC) * 1024)),
                                                     16, 0, 0);
                }
            }
            if (kc == 0) {
                float* bdst = (float*)(smem + LL.bias) + (hl & 1) * LL.TSP;
                for (int i0 = j * 64; i0 < LL.TSP; i0 += kLL * 64) {
                    const int i = i0 + lane;
                    const float* src = table + (i < g.table_size ? i * g.heads + h : 0);
                    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(bdst + i0), 4, 0, 0);
                }
                float* qdst = (float*)(smem + LL.bqkv) + (hl & 1) * LL.BQP;
                for (int i0 = j * 64; i0 < LL.BQP; i0 += kLL * 64) {
                    const int i = i0 + lane < F ? i0 + lane : 0;
                    const float* src = bqkv + (i / D) * C + h * D + i % D;
                    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(qdst + i0), 4, 0, 0);
                }
            }
        };
        // vector-memory operations of a wave complete in order: with stages up to
        // s + kLStages - 1 issued, stage s + 1 has landed once at most the copies of
        // the stages after it remain
        for (int s = 0; s < NS - 1; s++) issue(s);
        {
            int later = 0;
            for (int t = 1; t < NS - 1; t++) later += copies(t);
            wait_vmcnt_le(later);
        }
        loader_barrier(); // prologue
        for (int s = 0; s < steps; s++) {
            issue(s + NS - 1); // into the slot read in step s - 1
            int later = 0;
            for (int t = s + 2; t <= s + NS - 1; t++) later += copies(t);
            wait_vmcnt_le(later);
            loader_barrier(); // stage s done with, stage s + 1 landed
            if (s % KS == KS - 1) loader_barrier(); // the head's O in LDS
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        return;
    }

    // ---- compute waves
    const StreamLds L = stream_view(LL);
    const int col = lane & 15, grp = lane >> 4;
    const int wf = wave % WF, wt = wave / WF;
    const int t0 = wt * KT / WT, nt = (wt + 1) * KT / WT - t0; // this wave's token tiles
    const __amdgpu_buffer_rsrc_t ors =
        __builtin_amdgcn_make_buffer_rsrc((void*)o, 0, (int)((uint64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2] *
                                                                   (uint32_t)C * 2),
                                          kBufferWord3);
    lds_barrier(); // prologue
    f32x4 acc[FTW][TTW];
    for (int s = 0; s < steps; s++) {
        const int hl = s / KS, kc = s - hl * KS, h = h0 + hl;
        if (kc == 0) { // a head starts from zero (the sums are dead during the attention)
#pragma unroll
            for (int a = 0; a < FTW; a++)
#pragma unroll
                for (int b = 0; b < TTW; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const uint16_t* sx = (const uint16_t*)(smem + LL.ring + (s % NS) * LL.stage);
        const uint16_t* sw = sx + NP * kLK;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ks++) {
            bf16x8 fx[TTW];
#pragma unroll
            for (int b = 0; b < TTW; b++) {
                const int r = (t0 + (b < nt ? b : 0)) * 16 + col;
                fx[b] = *(const bf16x8*)&sx[r * kLK + k_slot<kLK>(r, ks * 4 + grp) * 8];
            }
#pragma unroll
            for (int a = 0; a < FTW; a++) {
                const int r = (wf * FTW + a) * 16 + col;
                const bf16x8 fw = *(const bf16x8*)&sw[r * kLK + k_slot<kLK>(r, ks * 4 + grp) * 8];
#pragma unroll
                for (int b = 0; b < TTW; b++)
                    if (b < nt) acc[a][b] = mfma32(fw, fx[b], acc[a][b]);
            }
        }
        if (kc == KS - 1) {
            // the head's q, k, v: + bias in fp32, one rounding to bf16, lane (col, grp)
            // writing features 4 grp .. 4 grp + 3 of a feature tile for token col
            const float* bq = (const float*)(smem + LL.bqkv) + (hl & 1) * LL.BQP;
#pragma unroll
            for (int a = 0; a < FTW; a++) {
                const int f = (wf * FTW + a) * 16 + 4 * grp;
                const int part = f / D, d = f - part * D;
                unsigned char* buf = smem + LL.q + part * LL.tb;
                const f32x4 bv = *(const f32x4*)&bq[f];
#pragma unroll
                for (int b = 0; b < TTW; b++) {
                    if (b < nt) {
                        const int n = (t0 + b) * 16 + col;
                        const f32x4 v = acc[a][b];
                        *(u32x2*)(buf + n * D * 2 + k_slot<D>(n, d >> 3) * 16 + (d & 7) * 2) =
                            u32x2{pack_bf16x2(v[0] + bv[0], v[1] + bv[1]), pack_bf16x2(v[2] + bv[2], v[3] + bv[3])};
                    }
                }
            }
        }
        lds_barrier(); // stage s done with; stage s + 1 landed; q, k, v complete after a head's last stage
        if (kc == KS - 1) {
            const uint32_t uu = wi * (uint32_t)g.heads + (uint32_t)h;
            for (int qi = 0; qi < QT; qi++) {
                const int qt = wave + qi * kLC;
                if (qt >= KT) break;
                BiasOffsets<KT, BIAS_VEC> bo;
                TileState<KT> ts;
                bias_offsets<KT, BIAS_VEC>(g, L, smem, qt, lane, bo);
                stream_qk<D, KT, BIAS_VEC>(g, L, smem, qt, lane, uu, hl & 1, 0, bo, ts);
                stream_pv<D, KT>(L, smem, lane, 0, ts);
            }
            lds_barrier(); // the head's O in LDS
            // O's token rows of head h: D / 8 lanes per row, 16 bytes each
            constexpr int LPR = D / 8, RPI = 64 / LPR, NI = NP / RPI;
            const uint16_t* Os = (const uint16_t*)(smem + LL.q);
            for (int i = wave; i < NI; i += kLC) {
                const int m = i * RPI + lane / LPR, c = lane % LPR;
                const u32x4 val = *(const u32x4*)(Os + m * D + k_slot<D>(m, c) * 8);
                const int r = (tw[m] & kRowMask) - 1;
                const uint32_t ob = r >= 0 ? ((uint32_t)r * (uint32_t)C + h * D + c * 8) * 2 : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b128(val, ors, ob, 0, kNonTemporal);
            }
        }
    }
}

typedef void (*layer_kernel_t)(Geometry, int, const uint16_t*, const uint16_t*, const float*, const float*,
                               uint16_t*);

// Windows of up to 9 query tiles (144 tokens); 128-wide heads up to 5 (the
// LDS of 3 ring stages and q, k, v).  Every tile count has its own variant.
template <int D, bool BV, int NS>
layer_kernel_t layer_variant_b(int KT) {
    constexpr int lo = layer_min_stages<layer_stage_channels<D>()>();
    if constexpr (NS < lo || NS > lo + 1) {
        return nullptr;
    } else {
    switch (KT) {
    case 1: return layer_qkv_attn_kernel<D, 1, BV, NS>;
    case 2: return layer_qkv_attn_kernel<D, 2, BV, NS>;
    case 3: return layer_qkv_attn_kernel<D, 3, BV, NS>;
    case 4: return layer_qkv_attn_kernel<D, 4, BV, NS>;
    case 5: return layer_qkv_attn_kernel<D, 5, BV, NS>;
    }
    if constexpr (D < 128) {
        switch (KT) {
        case 6: return layer_qkv_attn_kernel<D, 6, BV, NS>;
        case 7: return layer_qkv_attn_kernel<D, 7, BV, NS>;
        case 8: return layer_qkv_attn_kernel<D, 8, BV, NS>;
        case 9: return layer_qkv_attn_kernel<D, 9, BV, NS>;
        }
    }
    return nullptr;
    }
}

template <int NS>
layer_kernel_t layer_variant_ns(int D, bool bv, int KT) {
    if (D == 32) return bv ? layer_variant_b<32, true, NS>(KT) : layer_variant_b<32, false, NS>(KT);
    if (D == 64) return bv ? layer_variant_b<64, true, NS>(KT) : layer_variant_b<64, false, NS>(KT);
    if (D == 128) return bv ? layer_variant_b<128, true, NS>(KT) : layer_variant_b<128, false, NS>(KT);
    return nullptr;
}

int layer_channels(const Geometry& g) { return g.head_dim == 128 ? 32 : 64; }
int layer_min_stages_of(const Geometry& g) { return layer_channels(g) == 64 ? 2 : 3; }

// The deepest ring that fits the LDS, the minimum or one more, and that a
// head's stages fill (a head's first stage is issued into the slot of the
// previous head's bias only after that head's attention: stages per head >=
// slots - 1).
int layer_stages(const Geometry& g) {
    const int lo = layer_min_stages_of(g);
    const int ks = g.row / layer_channels(g);
    return layer_lds(g, lo + 1, layer_channels(g)).total <= (size_t)kLdsBytes && ks >= lo ? lo + 1 : lo;
}

layer_kernel_t layer_variant(const Geometry& g) {
    const int KT = (g.N + 15) / 16;
    const bool bv = g.win[2] % 4 == 0;
    switch (layer_stages(g)) {
    case 2: return layer_variant_ns<2>(g.head_dim, bv, KT);
    case 3: return layer_variant_ns<3>(g.head_dim, bv, KT);
    case 4: return layer_variant_ns<4>(g.head_dim, bv, KT);
    }
    return nullptr;
}

// Heads per workgroup: SWA_LAYER_HEADS when it divides the head count, else 1.
int layer_heads_per_group(const Geometry& g) {
    return g.heads % SWA_LAYER_HEADS == 0 ? SWA_LAYER_HEADS : 1;
}

} // namespace

bool layer_fused_fits(const Geometry& g) {
    const int64_t rows = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    const int SK = layer_channels(g);
    return layer_variant(g) != nullptr && layer_lds(g, layer_min_stages_of(g), SK).total <= (size_t)kLdsBytes &&
           g.row % SK == 0 && g.row / SK >= layer_stages(g) - 1 && rows < kRowMask &&
           rows * g.row * 2 < (int64_t)kOutOfRange && g.windows * g.heads < ((int64_t)1 << 31);
}

hipError_t prepare_layer_kernels(int max_lds) {
    for (int D : {32, 64, 128})
        for (bool bv : {true, false})
            for (int KT = 1; KT <= 9; KT++)
                for (layer_kernel_t f : {layer_variant_ns<2>(D, bv, KT), layer_variant_ns<3>(D, bv, KT),
                                         layer_variant_ns<4>(D, bv, KT)}) {
                    if (!f) continue;
                    const hipError_t e =
                        hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
                    if (e != hipSuccess) return e;
                }
    return hipSuccess;
}

hipError_t launch_layer_qkv_attention(const Geometry& g, const uint16_t* x, const uint16_t* w_qkv,
                                      const float* b_qkv, const float* table, uint16_t* o, hipStream_t s) {
    const layer_kernel_t f = layer_variant(g);
    if (!f || !layer_fused_fits(g)) return hipErrorInvalidValue;
    const int HG = layer_heads_per_group(g);
    hipLaunchKernelGGL(f, dim3((unsigned)(g.windows * (g.heads / HG))), dim3(kLWaves * 64),
                       layer_lds(g, layer_stages(g), layer_channels(g)).total, s, g, HG, x, w_qkv, b_qkv, table, o);
    return hipGetLastError();
}

} // namespace swa
