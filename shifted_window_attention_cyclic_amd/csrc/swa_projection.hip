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
// bf16: 256 x 256 tiles of (feature, token), 8 waves of 128 features x 64
// tokens, 32-deep stages double-buffered in LDS (register-staged: the next
// stage's global loads are in flight while the current one is multiplied),
// bf16 MFMA with fp32 accumulation, bias added in fp32, one rounding to bf16.
// The product is formed transposed (features x tokens) so that each lane ends
// with four consecutive features of one token: 8-byte stores along the row.
// Tiles are dealt so that each XCD walks the feature tiles of a run of token
// tiles: a token tile is read from HBM once into that XCD's L2 and the weights
// stay resident there.
//
// fp32: a plain 64 x 64 VALU tile with fp32 accumulation.
#include "swa_device.h"

namespace swa {
namespace {

constexpr int kPT = 256;      // tokens per tile
constexpr int kPF = 256;      // output features per tile
constexpr int kPK = 32;       // reduction depth per stage
constexpr int kPThreads = 512;

struct ProjLds {
    uint16_t w[2][kPF * kPK];
    uint16_t x[2][kPT * kPK];
};

__global__ __launch_bounds__(kPThreads) void proj_bf16_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              const float* __restrict__ bias, int M, int N,
                                                              int K, int split, uint16_t* __restrict__ d0,
                                                              uint16_t* __restrict__ d1,
                                                              uint16_t* __restrict__ d2) {
    __shared__ ProjLds L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntiles = (N + kPF - 1) / kPF;
    const int64_t tiles = (int64_t)((M + kPT - 1) / kPT) * ntiles;
    const int64_t wi = xcd_work_index(blockIdx.x, tiles);
    const int f0 = (int)(wi % ntiles) * kPF;
    const int t0 = (int)(wi / ntiles) * kPT;
    const int wf = (wave >> 2) * 128; // this wave's features within the tile
    const int wt = (wave & 3) * 64;   // and tokens

    // staging: each thread moves two 16-byte chunks of the weight stage and two
    // of the token stage (rows of 32 bf16 = 4 chunks)
    int srow[2], sk[2];
    const uint16_t* wsrc[2];
    const uint16_t* xsrc[2];
    bool wok[2], xok[2];
    for (int i = 0; i < 2; i++) {
        const int c = tid + i * kPThreads;
        srow[i] = c >> 2;
        sk[i] = c & 3;
        wok[i] = f0 + srow[i] < N;
        xok[i] = t0 + srow[i] < M;
        wsrc[i] = w + (int64_t)(wok[i] ? f0 + srow[i] : 0) * K + sk[i] * 8;
        xsrc[i] = x + (int64_t)(xok[i] ? t0 + srow[i] : 0) * K + sk[i] * 8;
    }
    u32x4 rw[2], rx[2];
    auto load = [&](int k0) {
        for (int i = 0; i < 2; i++) {
            rw[i] = wok[i] ? *(const u32x4*)(wsrc[i] + k0) : u32x4{0, 0, 0, 0};
            rx[i] = xok[i] ? *(const u32x4*)(xsrc[i] + k0) : u32x4{0, 0, 0, 0};
        }
    };
    auto stage = [&](int s) {
        for (int i = 0; i < 2; i++) {
            const int off = srow[i] * kPK + k_slot<kPK>(srow[i], sk[i]) * 8;
            *(u32x4*)&L.w[s][off] = rw[i];
            *(u32x4*)&L.x[s][off] = rx[i];
        }
    };

    f32x4 acc[8][4];
    for (int a = 0; a < 8; a++)
        for (int b = 0; b < 4; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int col = lane & 15, grp = lane >> 4;
    const int KT = K / kPK;
    load(0);
    stage(0);
    __syncthreads();
    for (int kt = 0; kt < KT; kt++) {
        const int s = kt & 1;
        if (kt + 1 < KT) load((kt + 1) * kPK);
        bf16x8 fw[8], fx[4];
        for (int a = 0; a < 8; a++) {
            const int r = wf + a * 16 + col;
            fw[a] = *(const bf16x8*)&L.w[s][r * kPK + k_slot<kPK>(r, grp) * 8];
        }
        for (int b = 0; b < 4; b++) {
            const int r = wt + b * 16 + col;
            fx[b] = *(const bf16x8*)&L.x[s][r * kPK + k_slot<kPK>(r, grp) * 8];
        }
        for (int a = 0; a < 8; a++)
            for (int b = 0; b < 4; b++) acc[a][b] = mfma32(fw[a], fx[b], acc[a][b]);
        if (kt + 1 < KT) stage(s ^ 1);
        __syncthreads();
    }

    // lane holds features f..f+3 (rows 4*grp.. of each 16 x 16 block) of token col
    for (int a = 0; a < 8; a++) {
        const int f = f0 + wf + a * 16 + 4 * grp;
        if (f >= N) continue;
        const float b0 = bias[f], b1 = bias[f + 1], b2 = bias[f + 2], b3 = bias[f + 3];
        const int t = f / split, c = f - t * split;
        uint16_t* dst = t == 0 ? d0 : (t == 1 ? d1 : d2);
        for (int b = 0; b < 4; b++) {
            const int m = t0 + wt + b * 16 + col;
            if (m >= M) continue;
            const f32x4 v = acc[a][b];
            *(u32x2*)(dst + (int64_t)m * split + c) = u32x2{pack_bf16x2(v[0] + b0, v[1] + b1),
                                                            pack_bf16x2(v[2] + b2, v[3] + b3)};
        }
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
    return M >= 1 && M < ((int64_t)1 << 31) && N >= 4 && N % 4 == 0 && K >= kPK && K % kPK == 0 &&
           split >= 4 && split % 4 == 0 && N <= 3 * split;
}

hipError_t launch_projection(bool bf16, const void* x, const void* w, const float* bias, int64_t M, int N, int K,
                             int split, void* d0, void* d1, void* d2, hipStream_t s) {
    if (!projection_fits(M, N, K, split)) return hipErrorInvalidValue;
    if (bf16) {
        const int64_t tiles = ((M + kPT - 1) / kPT) * ((N + kPF - 1) / kPF);
        hipLaunchKernelGGL(proj_bf16_kernel, dim3((unsigned)tiles), dim3(kPThreads), 0, s, (const uint16_t*)x,
                           (const uint16_t*)w, bias, (int)M, N, K, split, (uint16_t*)d0, (uint16_t*)d1,
                           (uint16_t*)d2);
    } else {
        const int64_t tiles = ((M + kFT - 1) / kFT) * ((N + kFT - 1) / kFT);
        hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)tiles), dim3(256), 0, s, (const float*)x,
                           (const float*)w, bias, (int)M, N, K, split, (float*)d0, (float*)d1, (float*)d2);
    }
    return hipGetLastError();
}

} // namespace swa
