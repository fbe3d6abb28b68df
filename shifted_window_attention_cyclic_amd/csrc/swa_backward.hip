// Backward pass of shifted-window multi-head self-attention on gfx950.
//
// The pages train the model (TERRA page, abstract; Table V), so the layer
// needs the gradients of its forward pass.  Per (window, head) unit, with
// P = softmax(scale * Q K^T + B) over the visible keys and dO the gradient of
// the output:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(P * dP),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
//   dB[n, m] = dS[n, m], summed over windows and batch items into the table
//   entry that B[n, m] is read from.
// Every real token lies in exactly one window of the shifted partition, so
// its dQ, dK and dV come from one unit each and need no accumulation across
// workgroups.  The table gradient does: each unit writes its share (one
// slice of the table) to a workspace, and two small kernels add the shares
// up in a fixed order.  A unit's share is gathered, not scattered: each
// thread takes a table entry, i.e. a relative offset (query minus key), and
// sums dS over the key positions whose query at that offset lies in the
// window, in a fixed order, from the bf16 dS that pass 2 reads anyway.  The
// whole backward pass is therefore bitwise reproducible.
//
// Kernels:
//   attn_bf16_bwd_kernel  one workgroup per unit, windows of up to 9 query
//                         tiles.  Pass 1, a query tile per wave: recompute the
//                         logits and P on MFMA, dP^T = V dO^T, dS and
//                         dQ^T = K^T dS^T; P and dS go to LDS as [query][key]
//                         bf16.  Pass 2, a key tile per wave: dV^T = dO^T P and
//                         dK^T = Q^T dS, with the operands fetched by
//                         transposing LDS reads.  Then the unit's share of the
//                         table gradient, an entry per thread.
//   attn_f32_bwd_kernel   the fp32 counterpart: one thread per query, then one
//                         per key.
//   dtable_chunk_kernel,
//   dtable_sum_kernel     the table gradient: per-chunk sums over windows,
//                         then the sum of the chunks.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "swa_device.h"
#include "swa_geometry.h"

namespace swa {

constexpr int kBwdWaves = 9;        // one per 16-query tile of the largest window taken
constexpr int kBwdMaxTiles = 9;
constexpr int kDtableChunks = 64;   // first-stage sums of the table gradient

// ---- LDS of the bf16 backward workgroup
struct BwdLds {
    int NP;
    size_t qs, ks, vs, dos, pm, dsm, bias, tw, kb, total;
};

__host__ __device__ inline BwdLds bwd_lds(const Geometry& g) {
    BwdLds L;
    L.NP = (g.N + 15) / 16 * 16;
    const size_t t = (size_t)L.NP * g.head_dim * 2;           // one [NP][D] bf16 tile
    const size_t tab = ((size_t)g.table_size * 4 + 15) / 16 * 16;
    L.qs = 0;
    L.ks = L.qs + t;
    L.vs = L.ks + t;
    L.dos = L.vs + t;
    L.pm = L.dos + t;                                          // P, [query][key] bf16
    L.dsm = L.pm + (size_t)L.NP * L.NP * 2;                    // dS, [query][key] bf16
    L.bias = L.dsm + (size_t)L.NP * L.NP * 2;
    L.tw = L.bias + tab;
    L.kb = L.tw + (size_t)L.NP * 4;
    L.total = L.kb + ((size_t)L.NP * 2 + 15) / 16 * 16;
    return L;
}

// Transposing read of four 16-bit elements: lane s of each 16-lane group
// points at row 4 * (s / 4) ... of a 4 x 16 block (see the forward kernels);
// lane (col, grp) receives the four rows' elements of column col.
__device__ inline u32x2 tr_read(const unsigned char* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_void*)p));
}

template <int D, bool BIAS_VEC>
__global__ __launch_bounds__(kBwdWaves * 64) void attn_bf16_bwd_kernel(
    Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ table, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ dtab_units) {
    constexpr int THREADS = kBwdWaves * 64;
    constexpr int KSTEPS = D / 32, DT = D / 16, CH = D / 8, RPC = 64 / CH;
    constexpr int KB = kBwdMaxTiles;
    extern __shared__ __align__(16) unsigned char smem[];
    const BwdLds L = bwd_lds(g);
    const int N = g.N, NP = L.NP, KT = NP / 16;
    float* bias = (float*)(smem + L.bias);
    int* tw = (int*)(smem + L.tw);
    uint16_t* kb = (uint16_t*)(smem + L.kb);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;

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

    // ---- token table (packed word: source row + 1 | mask field << 28), key
    // bias offsets, this head's bias slice
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
            tw[n] = ((is_pad ? -1 : tok) + 1) | ((region | (is_pad ? 8 : 0)) << 28);
            kb[n] = (uint16_t)((l[0] * g.tdy + l[1]) * g.tdx + l[2]);
        } else {
            tw[n] = 15 << 28;
            kb[n] = BIAS_VEC ? 3 : 0; // keeps qb - kb (- 3) inside the table
        }
    }
    for (int i = tid; i < g.table_size; i += THREADS) bias[i] = table[(size_t)i * g.heads + h];
    __syncthreads();

    // ---- Q, K, V, dO of the window into LDS ([token][d], swizzled; pad rows copy
    // row 0: their weights are 0, and pad queries are excluded below)
    {
        const int ncopy = NP * CH / 64;
        const int m0 = lane / CH;
        const uint16_t* src[4] = {q, k, v, dout};
        const size_t dst[4] = {L.qs, L.ks, L.vs, L.dos};
        for (int c = wave; c < 4 * ncopy; c += kBwdWaves) {
            const int tsr = c / ncopy, cc = c - tsr * ncopy;
            const int r1 = tw[cc * RPC + m0] & kRowMask;
            const uint64_t off = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + h * D +
                                 copy_chunk<D>(cc * RPC + m0, lane) * 8;
            __builtin_amdgcn_global_load_lds((const void*)(src[tsr] + off), (lds_void*)(smem + dst[tsr] + cc * 1024),
                                             16, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); // this wave's copies have landed
    __syncthreads();

    const uint16_t* Qs = (const uint16_t*)(smem + L.qs);
    const uint16_t* Ks = (const uint16_t*)(smem + L.ks);
    const uint16_t* Vs = (const uint16_t*)(smem + L.vs);
    const uint16_t* dOs = (const uint16_t*)(smem + L.dos);
    // [token][d] tile, transposed 4 x 16 read: rows t0 + 4 grp + 0..3, d = 16 dt + col
    auto tr_tile = [&](size_t base, int t0, int dt) __attribute__((always_inline)) {
        const int row = t0 + grp * 4 + (col >> 2);
        const int d = dt * 16 + (col & 3) * 4;
        return tr_read(smem + base + row * (D * 2) + k_slot<D>(row, d >> 3) * 16 + (d & 7) * 2);
    };
    // [query][key] bf16 matrix, transposed 4 x 16 read: queries q0 + 4 grp + 0..3, key k0 + col
    auto tr_mat = [&](size_t base, int q0, int k0) __attribute__((always_inline)) {
        const int row = q0 + grp * 4 + (col >> 2);
        return tr_read(smem + base + (size_t)row * NP * 2 + (k0 + (col & 3) * 4) * 2);
    };

    // ---- pass 1: query tile qt = wave
    if (wave < KT) {
        const int qt = wave;
        const int n = qt * 16 + col;
        const int qword = tw[n];
        const unsigned qreg = (unsigned)qword >> 28;
        const int r = (qword & kRowMask) - 1;
        const float qvalid = r >= 0 ? 1.f : 0.f; // pad queries have no output, so no gradient
        int qb;
        if (n < N) {
            int lt, ly, lx;
            local_coords(g, n, lt, ly, lx);
            qb = ((lt * g.tdy + ly) * g.tdx + lx) + g.c0;
        } else {
            qb = g.table_size - 1; // largest qb keeps qb - kb inside the table
        }
        bf16x8 qf[KSTEPS], df[KSTEPS]; // B operands: query n, d = 32 ks + 8 grp + 0..7
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Qs + n * D + k_slot<D>(n, ks * 4 + grp) * 8));
            df[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(dOs + n * D + k_slot<D>(n, ks * 4 + grp) * 8));
        }
        // S^T = K Q^T and dP^T = V dO^T, tile by tile; lane: query n, keys 16 kt + 4 grp + 0..3
        f32x4 s[KB], dp[KB];
#pragma unroll
        for (int kt = 0; kt < KB; kt++) {
            if (kt < KT) {
                const int krow = kt * 16 + col;
                f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ks++) {
                    const int slot = k_slot<D>(krow, ks * 4 + grp) * 8;
                    a0 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(Ks + krow * D + slot)), qf[ks], a0);
                    a1 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(Vs + krow * D + slot)), df[ks], a1);
                }
                s[kt] = a0;
                dp[kt] = a1;
            }
        }
        // logits (natural units), mask, max
        int bidx[KB][4]; // table entry of each (query, key) pair of the lane
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KB; kt++) {
            if (kt < KT) {
                const int key0 = kt * 16 + grp * 4;
                if (BIAS_VEC) {
                    const int e0 = qb - (int)kb[key0]; // keys key0 + i share a window row: entries e0 - i
#pragma unroll
                    for (int i = 0; i < 4; i++) bidx[kt][i] = e0 - i;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) bidx[kt][i] = qb - (int)kb[key0 + i];
                }
                const int4 kr4 = *(const int4*)(tw + key0);
                const int kreg[4] = {kr4.x, kr4.y, kr4.z, kr4.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float lg = fmaf(s[kt][i], g.scale, bias[bidx[kt][i]]);
                    if ((masked_window || key0 + 16 > N) && ((unsigned)kreg[i] >> 28) != qreg) lg = -INFINITY;
                    s[kt][i] = lg;
                    mx = fmaxf(mx, lg);
                }
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mc = (mx == -INFINITY ? 0.f : mx) * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KB; kt++) {
            if (kt < KT) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    s[kt][i] = __builtin_amdgcn_exp2f(fmaf(s[kt][i], kLog2e, -mc));
                    sum += s[kt][i];
                }
            }
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        const float inv = sum > 0.f ? qvalid / sum : 0.f;
        // P, then D = rowsum(P * dP)
        float dsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KB; kt++) {
            if (kt < KT) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    s[kt][i] *= inv;
                    dsum = fmaf(s[kt][i], dp[kt][i], dsum);
                }
            }
        }
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        // dS = P * (dP - D); P and dS to LDS ([query][key] bf16)
        unsigned pk[KB][2];
        uint16_t* Pm = (uint16_t*)(smem + L.pm);
        uint16_t* dSm = (uint16_t*)(smem + L.dsm);
#pragma unroll
        for (int kt = 0; kt < KB; kt++) {
            if (kt < KT) {
                f32x4 ds;
#pragma unroll
                for (int i = 0; i < 4; i++) ds[i] = s[kt][i] * (dp[kt][i] - dsum);
                pk[kt][0] = pack_bf16x2(ds[0], ds[1]);
                pk[kt][1] = pack_bf16x2(ds[2], ds[3]);
                const int key0 = kt * 16 + grp * 4;
                *(u32x2*)(Pm + (size_t)n * NP + key0) =
                    u32x2{pack_bf16x2(s[kt][0], s[kt][1]), pack_bf16x2(s[kt][2], s[kt][3])};
                *(u32x2*)(dSm + (size_t)n * NP + key0) = u32x2{pk[kt][0], pk[kt][1]};
            }
        }
        // dQ^T = K^T dS^T: the forward's O^T = V^T P^T with K for V and dS for P
        f32x4 acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; dt++) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KB; kt += 2) {
            if (kt < KT) {
                const bool pair = kt + 1 < KT;
                const bf16x8 bop = __builtin_bit_cast(
                    bf16x8, u32x4{pk[kt][0], pk[kt][1], pair ? pk[kt + 1][0] : 0u, pair ? pk[kt + 1][1] : 0u});
#pragma unroll
                for (int dt = 0; dt < DT; dt++) {
                    const u32x2 lo = tr_tile(L.ks, kt * 16, dt);
                    const u32x2 hi = pair ? tr_tile(L.ks, (kt + 1) * 16, dt) : u32x2{0u, 0u};
                    acc[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]}), bop, acc[dt]);
                }
            }
        }
        if (r >= 0) {
            uint16_t* op = dq + (uint64_t)(uint32_t)r * (uint32_t)g.row + h * D + grp * 4;
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
                *(u32x2*)(op + dt * 16) = u32x2{pack_bf16x2(acc[dt][0] * g.scale, acc[dt][1] * g.scale),
                                                pack_bf16x2(acc[dt][2] * g.scale, acc[dt][3] * g.scale)};
        }
    }
    __syncthreads();

    // ---- pass 2: key tile wave; contraction over the queries in pairs of tiles
    if (wave < KT) {
        const int k0 = wave * 16;
        f32x4 av[DT], ak[DT]; // dV^T and dK^T: lane (key k0 + col, d = 16 dt + 4 grp + 0..3)
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            av[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            ak[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int q0 = 0; q0 < NP; q0 += 32) {
            const bool pair = q0 + 16 < NP;
            const u32x2 p_lo = tr_mat(L.pm, q0, k0), s_lo = tr_mat(L.dsm, q0, k0);
            const u32x2 p_hi = pair ? tr_mat(L.pm, q0 + 16, k0) : u32x2{0u, 0u};
            const u32x2 s_hi = pair ? tr_mat(L.dsm, q0 + 16, k0) : u32x2{0u, 0u};
            const bf16x8 bp = __builtin_bit_cast(bf16x8, u32x4{p_lo[0], p_lo[1], p_hi[0], p_hi[1]});
            const bf16x8 bs = __builtin_bit_cast(bf16x8, u32x4{s_lo[0], s_lo[1], s_hi[0], s_hi[1]});
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const u32x2 o_lo = tr_tile(L.dos, q0, dt), q_lo = tr_tile(L.qs, q0, dt);
                const u32x2 o_hi = pair ? tr_tile(L.dos, q0 + 16, dt) : u32x2{0u, 0u};
                const u32x2 q_hi = pair ? tr_tile(L.qs, q0 + 16, dt) : u32x2{0u, 0u};
                av[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{o_lo[0], o_lo[1], o_hi[0], o_hi[1]}), bp, av[dt]);
                ak[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}), bs, ak[dt]);
            }
        }
        const int m = k0 + col;
        const int r = (tw[m] & kRowMask) - 1;
        if (r >= 0) {
            const uint64_t base = (uint64_t)(uint32_t)r * (uint32_t)g.row + h * D + grp * 4;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                *(u32x2*)(dv + base + dt * 16) =
                    u32x2{pack_bf16x2(av[dt][0], av[dt][1]), pack_bf16x2(av[dt][2], av[dt][3])};
                *(u32x2*)(dk + base + dt * 16) =
                    u32x2{pack_bf16x2(ak[dt][0] * g.scale, ak[dt][1] * g.scale),
                          pack_bf16x2(ak[dt][2] * g.scale, ak[dt][3] * g.scale)};
            }
        }
    }

    // ---- this unit's share of the table gradient.  Entry e is the offset
    // (query minus key) d = coords(e) - (w - 1): the sum of dS[key + d][key]
    // over the keys whose query at that offset lies in the window (pairs that
    // are masked or involve pad hold dS = 0).  Two balanced stages when the
    // partial sums fit in the P region (free once pass 2 is done): per
    // (query row, key row, x offset) along x, then per entry over the rows.
    float* dst = dtab_units + (size_t)work * g.table_size;
    const uint16_t* dSm = (const uint16_t*)(smem + L.dsm);
    auto ds_at = [&](int n, int m) __attribute__((always_inline)) {
        return __builtin_bit_cast(float, (unsigned)dSm[(size_t)n * NP + m] << 16);
    };
    const int wx = g.win[2], R = g.win[0] * g.win[1]; // tokens per window row; rows (t, y) per window
    const int items = R * R * g.tdx;
    __syncthreads(); // pass 2 is done with P
    if ((size_t)items * 4 <= (size_t)NP * NP * 2) {
        float* part = (float*)(smem + L.pm);
        for (int it = tid; it < items; it += THREADS) {
            const int ex = it % g.tdx, rr = it / g.tdx;
            const int rk = rr % R, rq = rr / R;
            const int dx = ex - (wx - 1);
            const int n0 = rq * wx + dx, m0 = rk * wx;
            float acc = 0.f;
            for (int kx = dx < 0 ? -dx : 0; kx < wx - (dx > 0 ? dx : 0); kx++) acc += ds_at(n0 + kx, m0 + kx);
            part[it] = acc;
        }
        __syncthreads();
        for (int e = tid; e < g.table_size; e += THREADS) {
            const int et = e / (g.tdy * g.tdx), r0 = e - et * (g.tdy * g.tdx);
            const int ey = r0 / g.tdx, ex = r0 - ey * g.tdx;
            const int dt = et - (g.win[0] - 1), dy = ey - (g.win[1] - 1);
            float acc = 0.f;
            for (int kt = dt < 0 ? -dt : 0; kt < g.win[0] - (dt > 0 ? dt : 0); kt++)
                for (int ky = dy < 0 ? -dy : 0; ky < g.win[1] - (dy > 0 ? dy : 0); ky++) {
                    const int rq = (kt + dt) * g.win[1] + ky + dy, rk = kt * g.win[1] + ky;
                    acc += part[(rq * R + rk) * g.tdx + ex];
                }
            dst[e] = acc;
        }
    } else {
        for (int e = tid; e < g.table_size; e += THREADS) {
            const int et = e / (g.tdy * g.tdx), r0 = e - et * (g.tdy * g.tdx);
            const int ey = r0 / g.tdx, ex = r0 - ey * g.tdx;
            const int dt = et - (g.win[0] - 1), dy = ey - (g.win[1] - 1), dx = ex - (wx - 1);
            float acc = 0.f;
            for (int kt = dt < 0 ? -dt : 0; kt < g.win[0] - (dt > 0 ? dt : 0); kt++)
                for (int ky = dy < 0 ? -dy : 0; ky < g.win[1] - (dy > 0 ? dy : 0); ky++) {
                    const int m0 = (kt * g.win[1] + ky) * wx;
                    const int n0 = ((kt + dt) * g.win[1] + ky + dy) * wx + dx;
                    for (int kx = dx < 0 ? -dx : 0; kx < wx - (dx > 0 ? dx : 0); kx++)
                        acc += ds_at(n0 + kx, m0 + kx);
                }
            dst[e] = acc;
        }
    }
}

// ---- fp32 backward: one block per unit, a thread per query, then per key
constexpr int kF32BwdThreads = 256;

__host__ __device__ inline size_t f32_bwd_lds_bytes(const Geometry& g) {
    return (size_t)g.N * g.head_dim * 4 * sizeof(float) + (size_t)g.N * g.N * 2 * sizeof(float) +
           (size_t)g.table_size * sizeof(float) + (size_t)g.N * 3 * sizeof(int);
}

template <int D>
__global__ __launch_bounds__(kF32BwdThreads) void attn_f32_bwd_kernel(
    Geometry g, const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ table, const float* __restrict__ dout, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dtab_units) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int N = g.N;
    float* Qs = (float*)smem;
    float* Ks = Qs + N * D;
    float* Vs = Ks + N * D;
    float* dOs = Vs + N * D;
    float* Pm = dOs + N * D;
    float* dSm = Pm + N * N;
    float* bias = dSm + N * N;
    int* kword = (int*)(bias + g.table_size);
    int* qword = kword + N;
    int* rowi = qword + N;

    const int64_t total = g.windows * g.heads;
    const int64_t work = xcd_work_index(blockIdx.x, total);
    const int64_t wi = work / g.heads;
    const int h = (int)(work - wi * g.heads);

    fill_token_tables(g, wi, false, N, kword, qword, rowi);
    for (int i = threadIdx.x; i < g.table_size; i += blockDim.x) bias[i] = table[(int64_t)i * g.heads + h];
    __syncthreads();
    for (int i = threadIdx.x; i < N * D; i += blockDim.x) {
        const int m = i / D, e = i % D;
        const int r = rowi[m];
        float a = 0.f, bb = 0.f, c = 0.f, d = 0.f;
        if (r >= 0) {
            const int64_t off = (int64_t)r * g.row + (int64_t)h * D + e;
            a = q[off];
            bb = k[off];
            c = v[off];
            d = dout[off];
        }
        Qs[i] = a;
        Ks[i] = bb;
        Vs[i] = c;
        dOs[i] = d;
    }
    __syncthreads();

    for (int n = threadIdx.x; n < N; n += blockDim.x) {
        float* prow = Pm + n * N;
        float* srow = dSm + n * N;
        const int qw = qword[n];
        if (rowi[n] < 0) { // pad query: no output, no gradient
            for (int m = 0; m < N; m++) prow[m] = srow[m] = 0.f;
            continue;
        }
        float mx = -INFINITY;
        for (int m = 0; m < N; m++) {
            const int kw = kword[m];
            float s = -INFINITY;
            if (visible(qw, kw)) {
                float dot = 0.f;
                for (int e = 0; e < D; e++) dot = fmaf(Qs[n * D + e], Ks[m * D + e], dot);
                s = dot * g.scale + bias[(qw & 0xFFFF) - (kw & 0xFFFF)];
            }
            prow[m] = s;
            mx = fmaxf(mx, s);
        }
        float den = 0.f;
        for (int m = 0; m < N; m++) {
            const float p = prow[m] == -INFINITY ? 0.f : expf(prow[m] - mx);
            prow[m] = p;
            den += p;
        }
        const float inv = 1.f / den;
        float dd = 0.f;
        for (int m = 0; m < N; m++) {
            const float p = prow[m] * inv;
            prow[m] = p;
            float dp = 0.f;
            if (p != 0.f)
                for (int e = 0; e < D; e++) dp = fmaf(dOs[n * D + e], Vs[m * D + e], dp);
            srow[m] = dp;
            dd = fmaf(p, dp, dd);
        }
        float acc[D];
        for (int e = 0; e < D; e++) acc[e] = 0.f;
        for (int m = 0; m < N; m++) {
            const float ds = prow[m] * (srow[m] - dd);
            srow[m] = ds;
            if (ds != 0.f)
                for (int e = 0; e < D; e++) acc[e] = fmaf(ds, Ks[m * D + e], acc[e]);
        }
        float* o = dq + (int64_t)rowi[n] * g.row + (int64_t)h * D;
        for (int e = 0; e < D; e++) o[e] = acc[e] * g.scale;
    }
    __syncthreads();

    for (int m = threadIdx.x; m < N; m += blockDim.x) {
        if (rowi[m] < 0) continue;
        float av[D], ak[D];
        for (int e = 0; e < D; e++) av[e] = ak[e] = 0.f;
        for (int n = 0; n < N; n++) {
            const float p = Pm[n * N + m], ds = dSm[n * N + m];
            for (int e = 0; e < D; e++) {
                av[e] = fmaf(p, dOs[n * D + e], av[e]);
                ak[e] = fmaf(ds, Qs[n * D + e], ak[e]);
            }
        }
        const int64_t off = (int64_t)rowi[m] * g.row + (int64_t)h * D;
        for (int e = 0; e < D; e++) {
            dv[off + e] = av[e];
            dk[off + e] = ak[e] * g.scale;
        }
    }
    // this unit's share of the table gradient, an entry per thread (see the bf16 kernel)
    float* dst = dtab_units + (size_t)work * g.table_size;
    for (int e = threadIdx.x; e < g.table_size; e += blockDim.x) {
        const int et = e / (g.tdy * g.tdx), r0 = e - et * (g.tdy * g.tdx);
        const int ey = r0 / g.tdx, ex = r0 - ey * g.tdx;
        const int dt = et - (g.win[0] - 1), dy = ey - (g.win[1] - 1), dx = ex - (g.win[2] - 1);
        float acc = 0.f;
        for (int kt = dt < 0 ? -dt : 0; kt < g.win[0] - (dt > 0 ? dt : 0); kt++)
            for (int ky = dy < 0 ? -dy : 0; ky < g.win[1] - (dy > 0 ? dy : 0); ky++) {
                const int m0 = (kt * g.win[1] + ky) * g.win[2];
                const int n0 = ((kt + dt) * g.win[1] + ky + dy) * g.win[2] + dx;
                for (int kx = dx < 0 ? -dx : 0; kx < g.win[2] - (dx > 0 ? dx : 0); kx++)
                    acc += dSm[(n0 + kx) * N + m0 + kx];
            }
        dst[e] = acc;
    }
}

// ---- the table gradient: dtable[e][h] = sum over windows (and batch) of the
// units' shares, in chunks of windows and then over the chunks, in order
__global__ __launch_bounds__(256) void dtable_chunk_kernel(int64_t windows, int heads, int ts,
                                                           const float* __restrict__ units,
                                                           float* __restrict__ chunks) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x; // h * ts + e
    if (idx >= heads * ts) return;
    const int c = blockIdx.y;
    const int64_t w0 = windows * c / kDtableChunks, w1 = windows * (c + 1) / kDtableChunks;
    float acc = 0.f;
    for (int64_t w = w0; w < w1; w++) acc += units[(size_t)w * heads * ts + idx];
    chunks[(size_t)c * heads * ts + idx] = acc;
}

__global__ __launch_bounds__(256) void dtable_sum_kernel(int heads, int ts, const float* __restrict__ chunks,
                                                         float* __restrict__ dtable) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x; // h * ts + e
    if (idx >= heads * ts) return;
    float acc = 0.f;
    for (int c = 0; c < kDtableChunks; c++) acc += chunks[(size_t)c * heads * ts + idx];
    const int h = idx / ts, e = idx - h * ts;
    dtable[(size_t)e * heads + h] = acc;
}

// ---- host side
bool backward_fits(const Geometry& g, bool bf16) {
    if (!bf16) return g.head_dim <= 64 && f32_bwd_lds_bytes(g) <= (size_t)kLdsBytes;
    const int64_t rows = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    return (g.N + 15) / 16 <= kBwdMaxTiles && bwd_lds(g).total <= (size_t)kLdsBytes && rows < kRowMask;
}

size_t backward_workspace_bytes(const Geometry& g) {
    const size_t units = (size_t)(g.windows * g.heads) * g.table_size;
    const size_t chunks = (size_t)kDtableChunks * g.heads * g.table_size;
    return (units + chunks) * sizeof(float);
}

typedef void (*bwd_bf16_t)(Geometry, const uint16_t*, const uint16_t*, const uint16_t*, const float*,
                           const uint16_t*, uint16_t*, uint16_t*, uint16_t*, float*);

static bwd_bf16_t bwd_bf16_variant(const Geometry& g) {
    const bool bv = g.win[2] % 4 == 0;
    if (g.head_dim == 32) return bv ? attn_bf16_bwd_kernel<32, true> : attn_bf16_bwd_kernel<32, false>;
    if (g.head_dim == 128) return bv ? attn_bf16_bwd_kernel<128, true> : attn_bf16_bwd_kernel<128, false>;
    return bv ? attn_bf16_bwd_kernel<64, true> : attn_bf16_bwd_kernel<64, false>;
}

hipError_t prepare_backward_kernels(int max_lds) {
    const void* fs[] = {(const void*)attn_bf16_bwd_kernel<32, true>,  (const void*)attn_bf16_bwd_kernel<32, false>,
                        (const void*)attn_bf16_bwd_kernel<64, true>,  (const void*)attn_bf16_bwd_kernel<64, false>,
                        (const void*)attn_bf16_bwd_kernel<128, true>, (const void*)attn_bf16_bwd_kernel<128, false>,
                        (const void*)attn_f32_bwd_kernel<32>,         (const void*)attn_f32_bwd_kernel<64>};
    for (const void* f : fs) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_backward(const Geometry& g, bool bf16, const void* q, const void* k, const void* v,
                           const float* table, const void* dout, void* dq, void* dk, void* dv, float* dtable,
                           void* workspace, hipStream_t s) {
    const dim3 grid((unsigned)(g.windows * g.heads));
    float* units = (float*)workspace;
    float* chunks = units + (size_t)(g.windows * g.heads) * g.table_size;
    if (bf16) {
        hipLaunchKernelGGL(bwd_bf16_variant(g), grid, dim3(kBwdWaves * 64), bwd_lds(g).total, s, g,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, table, (const uint16_t*)dout,
                           (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, units);
    } else if (g.head_dim == 32) {
        hipLaunchKernelGGL(attn_f32_bwd_kernel<32>, grid, dim3(kF32BwdThreads), f32_bwd_lds_bytes(g), s, g,
                           (const float*)q, (const float*)k, (const float*)v, table, (const float*)dout, (float*)dq,
                           (float*)dk, (float*)dv, units);
    } else {
        hipLaunchKernelGGL(attn_f32_bwd_kernel<64>, grid, dim3(kF32BwdThreads), f32_bwd_lds_bytes(g), s, g,
                           (const float*)q, (const float*)k, (const float*)v, table, (const float*)dout, (float*)dq,
                           (float*)dk, (float*)dv, units);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = g.heads * g.table_size;
    hipLaunchKernelGGL(dtable_chunk_kernel, dim3((n + 255) / 256, kDtableChunks), dim3(256), 0, s, g.windows,
                       g.heads, g.table_size, (const float*)units, chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(dtable_sum_kernel, dim3((n + 255) / 256), dim3(256), 0, s, g.heads, g.table_size,
                       (const float*)chunks, dtable);
    return hipGetLastError();
}

} // namespace swa
