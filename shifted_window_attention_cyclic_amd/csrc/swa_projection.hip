// The linear projections of a Swin block around the window attention (TERRA
// page, abstract: the models are stacks of Swin blocks; Table V: embedding
// width d = N_h heads x 128): every token's C = heads * head_dim channels are
// mapped to its queries, keys and values, and the attended values back to C
// channels.  Both are one product
//
//     out[m][n] = sum_k x[m][k] * w[n][k] + bias[n]
//
// over all tokens m, with w in a linear layer's [out_features][in_features]
// layout.  Output column n goes to tensor n / split, column n % split, so the
// query/key/value product writes the three tensors the attention reads
// ([token][heads][head_dim]) directly.
//
// bf16: 256 x 256 tiles of (feature, token), bf16 MFMA with fp32
// accumulation, bias added in fp32, one rounding to bf16.  A workgroup is
// persistent: it walks its tiles' 32-deep reduction stages as one stream, so
// the next tile's first stages load while the current tile finishes.  Four
// loader waves copy each stage (256 x 32 weights and 256 x 32 tokens) straight
// into a three-stage LDS ring with global_load_lds, two stages ahead, with the
// tile's biases alongside; eight compute waves (128 features x 64 tokens each)
// only read LDS, issue MFMAs and store.  The product is formed transposed
// (features x tokens): a lane ends with four consecutive features of one
// token.  A finished tile goes out through a small per-wave LDS staging area,
// sixteen tokens at a time, so that every store moves 16 bytes per lane and a
// wave's stores cover whole token rows (8-byte stores scattered over 16 rows
// cost the memory pipeline several times more per byte).  Tiles are dealt so
// that each XCD walks a contiguous run of work items.  When the weights fit
// L2 the feature tile runs fastest: a token tile is read from HBM once into
// that XCD's L2 and the weights stay resident there.  Larger weights (C = 8192:
// 400 MB) are walked in groups of 8 token tiles, so that the blocks running
// together share each weight slice 8 ways instead of re-reading it per token
// tile.
//
// fp32: a plain 64 x 64 VALU tile with fp32 accumulation.
#include "swa_device.h"
#include "swa_projection.h"

namespace swa {
namespace {

constexpr int kPT = 256;     // tokens per tile
constexpr int kPF = 256;     // output features per tile
constexpr int kPK = 32;      // reduction depth per stage
constexpr int kPStages = 3;  // LDS ring; stages are copied kPStages - 1 ahead
constexpr int kPCompute = 8; // compute waves
constexpr int kPLoaders = 4; // loader waves
constexpr int kPThreads = (kPCompute + kPLoaders) * 64;
constexpr int kPHalf = kPF * kPK * 2;  // bytes of one stage's weights (and of its tokens)
constexpr int kPStageBytes = 2 * kPHalf;
constexpr int kPBias0 = kPStages * kPStageBytes; // tile biases: tile ti in slot ti % 4
constexpr int kPBiasSlots = 4;
constexpr int kPStg0 = kPBias0 + kPBiasSlots * kPF * 4;
constexpr int kPStgRow = 128 * 2 + 32; // staging row: a wave's 128 features, padded against bank conflicts
constexpr int kPStgBytes = 16 * kPStgRow; // per compute wave: sixteen tokens (one 16 x 16 block row)
constexpr int kPLdsBytes = kPStg0 + kPCompute * kPStgBytes;
constexpr int kPCopies = kPHalf / 1024 / kPLoaders; // 1 KB copies per loader wave and operand per stage
static_assert(kPT == kPF, "weights and tokens share the stage layout");

// s_waitcnt immediates: vmcnt(n), expcnt and lgkmcnt unconstrained
constexpr int kVmIssuedPerStage = 2 * kPCopies;

__device__ inline void proj_compute_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The loader waves' LDS writes are copies they have waited for with vmcnt; a
// release fence would make the compiler wait for every copy in flight.
__device__ inline void proj_loader_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kPThreads) void proj_bf16_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              const float* __restrict__ bias, int M, int N,
                                                              int K, int split, uint16_t* __restrict__ d0,
                                                              uint16_t* __restrict__ d1,
                                                              uint16_t* __restrict__ d2, int GM) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntf = (N + kPF - 1) / kPF;
    const int ntt = (M + kPT - 1) / kPT;
    // work item -> (token tile, feature tile), in groups of GM token tiles that
    // walk all feature tiles with the token tile fastest: the tiles a wave of
    // blocks runs together share weight slices GM ways and token slices
    // (blocks / GM) ways.  GM = 1: the feature tile fastest (weights that fit L2).
    auto tile_of = [&](int item, int& f0_, int& t0_) __attribute__((always_inline)) {
        const int gsz = GM * ntf;
        const int gi = item / gsz, j = item - gi * gsz;
        const int rows = ntt - gi * GM < GM ? ntt - gi * GM : GM;
        t0_ = (gi * GM + j % rows) * kPT;
        f0_ = (j / rows) * kPF;
    };
    const int tiles = ((M + kPT - 1) / kPT) * ntf;
    const int G = gridDim.x;
    const int mine = (tiles - 1 - (int)blockIdx.x) / G + 1; // the grid has at most `tiles` blocks
    const int KT = K / kPK;
    const int steps = mine * KT;
    // this block's tiles: work items base, base + G/8, ... (the grid is a multiple
    // of 8 blocks whenever a block has more than one tile)
    const int base = (int)xcd_work_index(blockIdx.x, tiles);
    const int stride = G / kXcds;

    if (wave >= kPCompute) {
        // loader: stage s -> ring slot s % kPStages; a lane copies 16 bytes of row
        // r = 16 * copy + lane / 4 into slot position lane % 4, which holds the
        // logical chunk (lane % 4) ^ ((r / 2) % 4) (the swizzle the readers use)
        const int lw = wave - kPCompute;
        auto issue = [&](int s) {
            uint8_t* slot = lds + (s % kPStages) * kPStageBytes;
            const bool past = s >= steps;
            s = past ? steps - 1 : s; // past the end: a harmless copy into a slot nobody reads
            const int ti = s / KT, kt = s - ti * KT;
            const int item = base + ti * stride;
            int f0, t0;
            tile_of(item, f0, t0);
            if (kt == 0 && !past) {
                // the tile's biases go with its first stage, into bias slot ti % 4: read
                // at its last step, not overwritten before tile ti + 4 starts loading
                // (4-byte copies: the bias vector is only 4-byte aligned)
                const int f = f0 + 64 * lw + lane;
                __builtin_amdgcn_global_load_lds((const void*)(bias + (f < N ? f : N - 1)),
                                                 (lds_void*)(lds + kPBias0 + (ti % kPBiasSlots) * kPF * 4 + lw * 256),
                                                 4, 0, 0);
            }
            for (int j = 0; j < kPCopies; j++) {
                const int blk = lw * kPCopies + j;
                const int r = blk * 16 + (lane >> 2);
                const int c = (lane & 3) ^ ((r >> 1) & 3);
                const int fr = f0 + r < N ? f0 + r : N - 1; // rows past the end: read a real row,
                const int tr = t0 + r < M ? t0 + r : M - 1; // whose products are never stored
                __builtin_amdgcn_global_load_lds((const void*)(w + (int64_t)fr * K + kt * kPK + c * 8),
                                                 (lds_void*)(slot + blk * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const void*)(x + (int64_t)tr * K + kt * kPK + c * 8),
                                                 (lds_void*)(slot + kPHalf + blk * 1024), 16, 0, 0);
            }
        };
        for (int s = 0; s < kPStages - 1; s++) issue(s);
        // vector-memory operations of a wave complete in order: with the stages
        // s .. s + kPStages - 2 issued, at most kPStages - 2 stages outstanding
        // means stage s landed (a bias copy only adds to its stage's count, so the
        // wait stays sufficient)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kPStages - 2) * kVmIssuedPerStage));
        proj_loader_barrier();
        for (int s = 0; s < steps; s++) {
            issue(s + kPStages - 1); // into the slot read in step s - 1
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((kPStages - 2) * kVmIssuedPerStage)); // stage s + 1 landed
            proj_loader_barrier();
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); // no copy may outlive the block's LDS
        return;
    }

    const int wf = (wave >> 2) * 128; // this wave's features within the tile
    const int wt = (wave & 3) * 64;   // and tokens
    const int col = lane & 15, grp = lane >> 4;
    f32x4 acc[8][4];
    for (int a = 0; a < 8; a++)
        for (int b = 0; b < 4; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    proj_compute_barrier();
    for (int s = 0; s < steps; s++) {
        const uint16_t* sw = (const uint16_t*)(lds + (s % kPStages) * kPStageBytes);
        const uint16_t* sx = sw + kPF * kPK;
        bf16x8 fx[4];
        for (int b = 0; b < 4; b++) {
            const int r = wt + b * 16 + col;
            fx[b] = *(const bf16x8*)&sx[r * kPK + k_slot<kPK>(r, grp) * 8];
        }
        for (int a = 0; a < 8; a++) {
            const int r = wf + a * 16 + col;
            const bf16x8 fw = *(const bf16x8*)&sw[r * kPK + k_slot<kPK>(r, grp) * 8];
            for (int b = 0; b < 4; b++) acc[a][b] = mfma32(fw, fx[b], acc[a][b]);
        }
        const int ti = s / KT;
        if (s - ti * KT == KT - 1) {
            // lane (col, grp) holds features 4*grp.. of each 16-feature block a for
            // token col of each 16-token block b.  A block row of 16 tokens at a time
            // goes through the wave's staging rows; each lane then stores 16 bytes
            // (8 features) of one token row, 16 lanes covering the row's 128 features.  The
            // biases come from LDS: a global load here would make the wave wait for
            // every store it has in flight (the memory counter is in order).
            const int item = base + ti * stride;
            int f0, t0;
            tile_of(item, f0, t0);
            const float* tb = (const float*)(lds + kPBias0 + (ti % kPBiasSlots) * kPF * 4);
            uint8_t* stg = lds + kPStg0 + wave * kPStgBytes;
            const int fq = f0 + wf + 8 * col; // the 8 features this lane stores
            const int tq = (fq >= split) + (fq >= 2 * split);
            uint16_t* dq = (tq == 0 ? d0 : (tq == 1 ? d1 : d2)) + (fq - tq * split);
            const bool fok = fq < N;
            for (int b = 0; b < 4; b++) {
                uint8_t* row = stg + col * kPStgRow;
                for (int a = 0; a < 8; a++) {
                    const f32x4 bv = *(const f32x4*)&tb[wf + a * 16 + 4 * grp];
                    const f32x4 v = acc[a][b];
                    *(u32x2*)(row + (a * 16 + 4 * grp) * 2) =
                        u32x2{pack_bf16x2(v[0] + bv[0], v[1] + bv[1]), pack_bf16x2(v[2] + bv[2], v[3] + bv[3])};
                }
                // LDS operations of a wave run in order: these reads see the writes
                // above, and the next block's writes follow them
                for (int j = 0; j < 4; j++) {
                    const int r = 4 * j + grp;
                    const u32x4 val = *(const u32x4*)(stg + r * kPStgRow + col * 16);
                    const int m = t0 + wt + b * 16 + r;
                    // non-temporal: the outputs are not read again here, and
                    // keeping them out of L2 keeps the token tiles and weights in it
                    if (fok && m < M) __builtin_nontemporal_store(val, (u32x4*)(dq + (int64_t)m * split));
                }
            }
            for (int a = 0; a < 8; a++)
                for (int b = 0; b < 4; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        proj_compute_barrier();
    }
}

constexpr int kFT = 64, kFK = 16;

__global__ __launch_bounds__(256) void proj_f32_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                       const float* __restrict__ bias, int M, int N, int K,
                                                       int split, float* __restrict__ d0, float* __restrict__ d1,
                                                       float* __restrict__ d2) {
    __shared__ float xs[kFK][kFT + 4];
    __shared__ float ws[kFK][kFT + 4];
    const int tid = threadIdx.x;
    const int ntiles = (N + kFT - 1) / kFT;
    const int f0 = (int)(blockIdx.x % ntiles) * kFT;
    const int t0 = (int)(blockIdx.x / ntiles) * kFT;
    const int tf = (tid & 15) * 4, tt = (tid >> 4) * 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kFK) {
        for (int i = 0; i < 4; i++) {
            const int e = tid + i * 256, r = e >> 4, kk = e & 15;
            const bool kin = k0 + kk < K;
            xs[kk][r] = kin && t0 + r < M ? x[(int64_t)(t0 + r) * K + k0 + kk] : 0.f;
            ws[kk][r] = kin && f0 + r < N ? w[(int64_t)(f0 + r) * K + k0 + kk] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < kFK; kk++) {
            float a[4], b[4];
            for (int i = 0; i < 4; i++) {
                a[i] = xs[kk][tt + i];
                b[i] = ws[kk][tf + i];
            }
            for (int i = 0; i < 4; i++)
                for (int j = 0; j < 4; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    for (int j = 0; j < 4; j++) {
        const int f = f0 + tf + j;
        if (f >= N) continue;
        const int t = f / split, c = f - t * split;
        float* dst = t == 0 ? d0 : (t == 1 ? d1 : d2);
        for (int i = 0; i < 4; i++) {
            const int m = t0 + tt + i;
            if (m < M) dst[(int64_t)m * split + c] = acc[i][j] + bias[f];
        }
    }
}

} // namespace

bool projection_fits(int64_t M, int N, int K, int split) {
    // tile and stage counts stay within 32 bits: at most 2^31 / 256 token tiles
    // times 2^15 / 256 feature tiles, times the stages of a tile
    return M >= 1 && M < ((int64_t)1 << 31) && N >= 8 && N % 8 == 0 && N <= (1 << 15) && K >= kPK &&
           K % kPK == 0 && K <= (1 << 16) && split >= 8 && split % 8 == 0 && N <= 3 * split;
}

namespace {

// Persistent blocks: one per compute unit, a multiple of 8 (the XCD count)
// whenever there are more tiles than blocks.  The LDS ring is set up once
// per device.
hipError_t projection_grid(int64_t tiles, int* grid) {
    constexpr int kMaxDevices = 64;
    static int cus[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (cus[dev] == 0) {
        e = hipFuncSetAttribute((const void*)proj_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kPLdsBytes);
        if (e != hipSuccess) return e;
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus[dev] = n > kXcds ? n / kXcds * kXcds : kXcds;
    }
    *grid = tiles <= cus[dev] ? (int)tiles : cus[dev];
    return hipSuccess;
}

} // namespace

hipError_t launch_projection(bool bf16, const void* x, const void* w, const float* bias, int64_t M, int N, int K,
                             int split, void* d0, void* d1, void* d2, hipStream_t s) {
    if (!projection_fits(M, N, K, split)) return hipErrorInvalidValue;
    if (bf16) {
        const int64_t tiles = ((M + kPT - 1) / kPT) * ((N + kPF - 1) / kPF);
        int grid = 0;
        hipError_t e = projection_grid(tiles, &grid);
        if (e != hipSuccess) return e;
        // weights beyond a couple of MB do not stay in an XCD's L2: group the tiles
        const int GM = (int64_t)N * K * 2 > ((int64_t)2 << 20) ? 8 : 1;
        hipLaunchKernelGGL(proj_bf16_kernel, dim3(grid), dim3(kPThreads), kPLdsBytes, s, (const uint16_t*)x,
                           (const uint16_t*)w, bias, (int)M, N, K, split, (uint16_t*)d0, (uint16_t*)d1,
                           (uint16_t*)d2, GM);
    } else {
        const int64_t tiles = ((M + kFT - 1) / kFT) * ((N + kFT - 1) / kFT);
        hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)tiles), dim3(256), 0, s, (const float*)x,
                           (const float*)w, bias, (int)M, N, K, split, (float*)d0, (float*)d1, (float*)d2);
    }
    return hipGetLastError();
}

} // namespace swa
