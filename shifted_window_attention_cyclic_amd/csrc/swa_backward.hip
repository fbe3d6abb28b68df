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
// single-workgroup backward pass is therefore bitwise reproducible.
//
// Kernels:
//   attn_bf16_bwd_pkernel windows of up to 9 query tiles: persistent
//                         workgroups, 9 compute waves that take unit after
//                         unit and 2 loader waves that copy the next unit's
//                         Q, K, V and dO into LDS as this one's are done with.
//                         Per unit (bwd_unit): pass 1, a query tile per wave:
//                         recompute the logits and P on MFMA, dP^T = V dO^T, dS
//                         and dQ^T = K^T dS^T; P and dS go to LDS as
//                         [query][key] bf16.  Pass 2, a key tile per wave:
//                         dV^T = dO^T P and dK^T = Q^T dS, with the operands
//                         fetched by transposing LDS reads.  Then the unit's
//                         share of the table gradient, gathered.
//   attn_bf16_bwd_kernel  the same per unit, one workgroup per unit, where the
//                         persistent kernel's LDS (second table and bias
//                         slots) does not fit.
//   attn_f32_bwd_kernel   the fp32 counterpart: one thread per query, then one
//                         per key.
//   attn_bf16_bwd_q_kernel, attn_bf16_bwd_kv_kernel, attn_bf16_bwd_kvp_kernel
//                         bf16 windows the single-workgroup kernel does not
//                         take (see below); the persistent key kernel
//                         attn_bf16_bwd_kvp_kernel where it fits (129 .. 288
//                         tokens, heads of 32 or 64), with pair_runs_kernel
//                         and dtable_pairs_kernel for its table gradient.
//   dtable_chunk_kernel,
//   dtable_sum_kernel     the table gradient: per-chunk sums over windows,
//                         then the sum of the chunks.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "swa_backward.h"
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

// Block barriers of a workgroup whose loader waves issue LDS copies while
// its compute waves read LDS.  The compute waves' barrier fences LDS only
// (they issue no copies, so nothing of theirs is in flight into LDS).  The
// loader waves' barrier has no release fence, which would make the compiler
// wait for every copy in flight; their only other LDS writes are table words
// (covered by the lgkmcnt wait), and the empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ inline void bwd_compute_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ inline void bwd_loader_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// unit -> head, batch item and window coordinates
struct BwdUnit {
    int h, b, wc[3];
};
__device__ inline BwdUnit bwd_decode(const Geometry& g, uint32_t work) {
    BwdUnit U;
    const uint32_t wi = fdiv(g.fd_heads, work);
    U.h = (int)(work - wi * (uint32_t)g.heads);
    U.b = (int)fdiv(g.fd_nW, wi);
    const uint32_t r = wi - (uint32_t)U.b * (uint32_t)g.nW;
    const uint32_t r2 = fdiv(g.fd_nwin2, r);
    U.wc[2] = (int)(r - r2 * (uint32_t)g.nwin[2]);
    U.wc[0] = (int)fdiv(g.fd_nwin1, r2);
    U.wc[1] = (int)(r2 - (uint32_t)U.wc[0] * (uint32_t)g.nwin[1]);
    return U;
}

// Token word of local token n of a window (batch item b, window coordinates
// wc): source row + 1 (0 for pad and for slots past N) | mask field << 28;
// and the token's key bias offset.
template <bool BIAS_VEC>
__device__ inline void bwd_token(const Geometry& g, int b, const int wc[3], int n, int& word, uint16_t& kbo) {
    if (n < g.N) {
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
        word = ((is_pad ? -1 : tok) + 1) | ((region | (is_pad ? 8 : 0)) << 28);
        kbo = (uint16_t)((l[0] * g.tdy + l[1]) * g.tdx + l[2]);
    } else {
        word = 15 << 28;
        kbo = BIAS_VEC ? 3 : 0; // keeps qb - kb (- 3) inside the table
    }
}

// Whether the table-gradient share is gathered in two stages: when the
// per-(query row, key row, x offset) partial sums fit the P region.
__host__ __device__ inline bool bwd_gather_staged(const Geometry& g) {
    const size_t R = (size_t)g.win[0] * g.win[1];
    const size_t NP = (size_t)(g.N + 15) / 16 * 16;
    return R * R * g.tdx * 4 <= NP * NP * 2;
}

// Pass 1, pass 2 and the table-gradient share of one unit whose Q, K, V and
// dO ([token][d], swizzled), token table tw, key bias offsets kb and bias
// slice are in LDS, into dq, dk, dv and the share dst.  Run by waves 0 ..
// kBwdWaves - 1; barrier() is the block barrier, which any other wave of the
// workgroup meets as often: twice, three times when bwd_gather_staged(g).
template <int D, bool BIAS_VEC, typename Barrier>
__device__ __forceinline__ void bwd_unit(const Geometry& g, unsigned char* smem, const BwdLds& L,
                                         const float* bias, const int* tw, const uint16_t* kb, int h,
                                         bool masked_window, uint16_t* __restrict__ dq, uint16_t* __restrict__ dk,
                                         uint16_t* __restrict__ dv, float* __restrict__ dst, Barrier&& barrier) {
    constexpr int THREADS = kBwdWaves * 64;
    constexpr int KSTEPS = D / 32, DT = D / 16;
    constexpr int KB = kBwdMaxTiles;
    const int N = g.N, NP = L.NP, KT = NP / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
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
    barrier(); // P and dS complete

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
    const uint16_t* dSm = (const uint16_t*)(smem + L.dsm);
    auto ds_at = [&](int n, int m) __attribute__((always_inline)) {
        return __builtin_bit_cast(float, (unsigned)dSm[(size_t)n * NP + m] << 16);
    };
    const int wx = g.win[2], R = g.win[0] * g.win[1]; // tokens per window row; rows (t, y) per window
    barrier(); // pass 2 is done with P
    if (bwd_gather_staged(g)) {
        float* part = (float*)(smem + L.pm);
        // A thread takes one (key row, x offset) and a share of the query rows,
        // so the integer divisions that place it happen once, not per sum;
        // neighbouring lanes take neighbouring key rows, whose reads sit a window
        // row apart in one dS row and so spread over the banks.
        const int cols = R * g.tdx;
        const int split = cols < THREADS ? THREADS / cols : 1;
        for (int t = tid; t < cols * split; t += THREADS) {
            const int rk = t % R, rest = t / R;
            const int ex = rest % g.tdx, first = rest / g.tdx;
            const int dx = ex - (wx - 1);
            const int lo = dx < 0 ? -dx : 0, hi = wx - (dx > 0 ? dx : 0);
            const int m0 = rk * wx;
            // the thread's query rows (up to G at a time, G the thread's row count
            // rounded up to 2, 4 or 8) share the loop over x, so their reads are
            // independent and in flight together; each sum still adds its terms in
            // x order
            auto rows = [&](auto gtag) __attribute__((always_inline)) {
                constexpr int G = decltype(gtag)::value;
                for (int rq0 = first; rq0 < R; rq0 += G * split) {
                    int n0[G];
                    float acc[G];
#pragma unroll
                    for (int u = 0; u < G; u++) {
                        const int rq = rq0 + u * split;
                        n0[u] = (rq < R ? rq : first) * wx + dx;
                        acc[u] = 0.f;
                    }
                    for (int kx = lo; kx < hi; kx++) {
                        float x[G];
#pragma unroll
                        for (int u = 0; u < G; u++) x[u] = ds_at(n0[u] + kx, m0 + kx);
#pragma unroll
                        for (int u = 0; u < G; u++) acc[u] += x[u];
                    }
#pragma unroll
                    for (int u = 0; u < G; u++) {
                        const int rq = rq0 + u * split;
                        if (rq < R) part[(rq * R + rk) * g.tdx + ex] = acc[u];
                    }
                }
            };
            const int most = (R - 1) / split + 1; // the most query rows a thread takes
            if (most <= 2)
                rows(std::integral_constant<int, 2>());
            else if (most <= 4)
                rows(std::integral_constant<int, 4>());
            else
                rows(std::integral_constant<int, 8>());
        }
        barrier(); // stage 1 complete
        for (int e = tid; e < g.table_size; e += THREADS) {
            const int et = e / (g.tdy * g.tdx), r0 = e - et * (g.tdy * g.tdx);
            const int ey = r0 / g.tdx, ex = r0 - ey * g.tdx;
            const int dt = et - (g.win[0] - 1), dy = ey - (g.win[1] - 1);
            // four reads in flight at a time, all issued: a step past the end
            // re-reads the last term and adds +0, which leaves the sum exact (a sum
            // that starts at +0 is never -0)
            const int ylo = dy < 0 ? -dy : 0, yhi = g.win[1] - (dy > 0 ? dy : 0);
            float acc = 0.f;
            for (int kt = dt < 0 ? -dt : 0; kt < g.win[0] - (dt > 0 ? dt : 0); kt++)
                for (int ky = ylo; ky < yhi; ky += 4) {
                    float x[4];
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const int yy = ky + u < yhi ? ky + u : yhi - 1;
                        const int rq = (kt + dt) * g.win[1] + yy + dy, rk = kt * g.win[1] + yy;
                        x[u] = part[(rq * R + rk) * g.tdx + ex];
                    }
#pragma unroll
                    for (int u = 0; u < 4; u++) acc += ky + u < yhi ? x[u] : 0.f;
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

// One workgroup per unit: the token table, the bias slice and the unit's Q,
// K, V and dO into LDS, then bwd_unit.
template <int D, bool BIAS_VEC>
__global__ __launch_bounds__(kBwdWaves * 64) void attn_bf16_bwd_kernel(
    Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ table, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ dtab_units, uint32_t work0,
    uint32_t count) {
    constexpr int THREADS = kBwdWaves * 64;
    constexpr int CH = D / 8, RPC = 64 / CH;
    extern __shared__ __align__(16) unsigned char smem[];
    const BwdLds L = bwd_lds(g);
    const int NP = L.NP;
    float* bias = (float*)(smem + L.bias);
    int* tw = (int*)(smem + L.tw);
    uint16_t* kb = (uint16_t*)(smem + L.kb);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // units work0 .. work0 + count - 1 (all of them, or one pass of the no-workspace entry)
    const uint32_t work = work0 + (uint32_t)xcd_work_index(blockIdx.x, count);
    const BwdUnit U = bwd_decode(g, work);

    for (int n = tid; n < NP; n += THREADS) {
        int word;
        uint16_t kbo;
        bwd_token<BIAS_VEC>(g, U.b, U.wc, n, word, kbo);
        tw[n] = word;
        kb[n] = kbo;
    }
    for (int i = tid; i < g.table_size; i += THREADS) bias[i] = table[(size_t)U.h * g.table_size + i];
    __syncthreads();

    // ---- Q, K, V, dO of the window into LDS ([token][d], swizzled; pad rows copy
    // row 0: their weights are 0, and pad queries are excluded)
    {
        const int ncopy = NP * CH / 64;
        const int m0 = lane / CH;
        const uint16_t* src[4] = {q, k, v, dout};
        const size_t dst[4] = {L.qs, L.ks, L.vs, L.dos};
        for (int c = wave; c < 4 * ncopy; c += kBwdWaves) {
            const int tsr = c / ncopy, cc = c - tsr * ncopy;
            const int r1 = tw[cc * RPC + m0] & kRowMask;
            const uint64_t off = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + U.h * D +
                                 copy_chunk<D>(cc * RPC + m0, lane) * 8;
            __builtin_amdgcn_global_load_lds((const void*)(src[tsr] + off), (lds_void*)(smem + dst[tsr] + cc * 1024),
                                             16, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); // this wave's copies have landed
    __syncthreads();
    bwd_unit<D, BIAS_VEC>(g, smem, L, bias, tw, kb, U.h, window_maybe_masked(g, U.wc), dq, dk, dv,
                          dtab_units + (size_t)(work - work0) * g.table_size, [] { bwd_compute_barrier(); });
}

// ---- the same computation in persistent workgroups (one per compute unit):
// 9 compute waves run bwd_unit on unit after unit, and two loader waves fill
// the LDS for the next unit behind them.  The next unit's token table and
// bias slice go to the other of two slots while the compute waves run pass 1;
// its K and V replace this unit's once pass 1 is done with them, its Q and dO
// once pass 2 is; the copies land while the table gradient is gathered.  The
// loader waves build the token words of the rows they copy themselves, so
// they need no barrier of their own.
constexpr int kBwdPLoaders = 2;

struct BwdPLds {
    BwdLds L;      // Q, K, V, dO, P and dS as in the one-shot kernel
    size_t bias, tw, kb, bias_stride, tw_stride, kb_stride, total; // slot 0 and slot strides
};

__host__ __device__ inline BwdPLds bwd_plds(const Geometry& g) {
    BwdPLds P;
    P.L = bwd_lds(g);
    P.bias_stride = ((size_t)g.table_size + 63) / 64 * 256; // whole 64-float copies
    P.tw_stride = (size_t)P.L.NP * 4;
    P.kb_stride = ((size_t)P.L.NP * 2 + 15) / 16 * 16;
    P.bias = P.L.bias;
    P.tw = P.bias + 2 * P.bias_stride;
    P.kb = P.tw + 2 * P.tw_stride;
    P.total = P.kb + 2 * P.kb_stride;
    return P;
}

template <int D, bool BIAS_VEC>
__global__ __launch_bounds__((kBwdWaves + kBwdPLoaders) * 64) void attn_bf16_bwd_pkernel(
    Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ table, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ dtab_units, uint32_t work0,
    uint32_t count) {
    constexpr int CH = D / 8, RPC = 64 / CH;
    extern __shared__ __align__(16) unsigned char smem[];
    const BwdPLds P = bwd_plds(g);
    const int NP = P.L.NP;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool staged = bwd_gather_staged(g);

    // units work0 + u, u = 0 .. count - 1: each XCD takes a contiguous range,
    // its workgroups in turn
    const uint32_t per = gridDim.x / kXcds, xcd = blockIdx.x % kXcds;
    const uint32_t uend = (uint32_t)((uint64_t)count * (xcd + 1) / kXcds);
    const uint32_t u0 = (uint32_t)((uint64_t)count * xcd / kXcds) + blockIdx.x / kXcds;
    if (u0 >= uend) return;

    if (wave >= kBwdWaves) {
        // ---- loader waves: copy cc = j, j + 2, ... of each tensor (RPC rows of
        // 1 KB each); the lanes of a row also write its token word and bias offset
        const int j = wave - kBwdWaves;
        constexpr int MAXC = (kBwdMaxTiles * 16 * CH / 64 + kBwdPLoaders - 1) / kBwdPLoaders;
        const int ncopy = NP * CH / 64;
        const int mine = (ncopy - j + kBwdPLoaders - 1) / kBwdPLoaders;
        uint64_t off[MAXC]; // source offsets of this wave's copies of the next unit
        auto prepare = [&](uint32_t u, int slot) __attribute__((always_inline)) {
            const BwdUnit U = bwd_decode(g, work0 + u);
            int* tws = (int*)(smem + P.tw + slot * P.tw_stride);
            uint16_t* kbs = (uint16_t*)(smem + P.kb + slot * P.kb_stride);
#pragma unroll
            for (int i = 0; i < MAXC; i++) {
                if (i < mine) {
                    const int n = (j + i * kBwdPLoaders) * RPC + lane / CH;
                    int word;
                    uint16_t kbo;
                    bwd_token<BIAS_VEC>(g, U.b, U.wc, n, word, kbo);
                    if (lane % CH == 0) {
                        tws[n] = word;
                        kbs[n] = kbo;
                    }
                    const int r1 = word & kRowMask;
                    off[i] = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + U.h * D +
                             copy_chunk<D>(n, lane) * 8;
                }
            }
            float* bs = (float*)(smem + P.bias + slot * P.bias_stride);
            for (int i0 = j * 64; i0 < g.table_size; i0 += kBwdPLoaders * 64) {
                const int i = i0 + lane;
                const float* src = table + (size_t)U.h * g.table_size + (i < g.table_size ? i : 0);
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(bs + i0), 4, 0, 0);
            }
        };
        auto issue = [&](const uint16_t* src, size_t dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < MAXC; i++)
                if (i < mine)
                    __builtin_amdgcn_global_load_lds((const void*)(src + off[i]),
                                                     (lds_void*)(smem + dst + (j + i * kBwdPLoaders) * 1024), 16, 0, 0);
        };
        prepare(u0, 0);
        issue(q, P.L.qs);
        issue(k, P.L.ks);
        issue(v, P.L.vs);
        issue(dout, P.L.dos);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        bwd_loader_barrier(); // the first unit is in LDS
        int it = 0;
        for (uint32_t u = u0; u < uend; u += per, it++) {
            const bool next = u + per < uend;
            if (next) prepare(u + per, (it + 1) & 1); // the slot the unit before this one used
            bwd_loader_barrier();                     // pass 1 done with K and V
            if (next) {
                issue(k, P.L.ks);
                issue(v, P.L.vs);
            }
            bwd_loader_barrier(); // pass 2 done with Q and dO
            if (next) {
                issue(q, P.L.qs);
                issue(dout, P.L.dos);
            }
            if (staged) bwd_loader_barrier(); // the gather's first stage
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            bwd_loader_barrier(); // the unit is done, the next one is in LDS
        }
        return;
    }

    bwd_compute_barrier(); // the first unit is in LDS
    int it = 0;
    for (uint32_t u = u0; u < uend; u += per, it++) {
        const int slot = it & 1;
        const BwdUnit U = bwd_decode(g, work0 + u);
        bwd_unit<D, BIAS_VEC>(g, smem, P.L, (const float*)(smem + P.bias + slot * P.bias_stride),
                              (const int*)(smem + P.tw + slot * P.tw_stride),
                              (const uint16_t*)(smem + P.kb + slot * P.kb_stride), U.h, window_maybe_masked(g, U.wc),
                              dq, dk, dv, dtab_units + (size_t)u * g.table_size, [] { bwd_compute_barrier(); });
        bwd_compute_barrier(); // the unit is done, the next one is in LDS
    }
}

// ---- bf16 backward for windows beyond the single-workgroup kernel (more than
// 9 query tiles, e.g. 2x12x12 or 32x32): nothing of size N x N is kept.  Two
// kernels, both streaming 32-token blocks of the other side through an LDS
// ring filled by loader waves of their own:
//   attn_bf16_bwd_q_kernel   a block of 64 or 128 queries (a wave per 16) of
//     a unit.  Two passes over the key blocks: first the softmax statistics
//     and D = rowsum(P * dP) together (running max, normaliser and D, the
//     last two rescaled whenever the max grows), then dS and
//     dQ^T = K^T dS^T.  The statistics (as log2 of the normaliser) and D go
//     to the workspace.
//   attn_bf16_bwd_kv_kernel  one workgroup per unit, a wave per 16-key tile
//     (K and V of the tile held as MFMA operands in registers).  Per block of
//     32 queries: S = Q K^T and dP = dO V^T, P from the stored statistics,
//     dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS; dS is added
//     into the unit's table-gradient share in LDS with atomics (so this share,
//     unlike the small-window kernel's, is summed in a run-dependent order).
// Only the loader waves issue LDS copies.  A wave that both copies and reads
// LDS gets a vmcnt(0) from the compiler before its barriers, transposing
// reads and LDS atomics (it cannot tell the copies in flight from the data
// read), which leaves no copy in flight while the wave computes.
constexpr int kBwdBlk = 32;     // tokens per streamed block
constexpr int kBwdStages = 3;   // ring slots: the block in use and two in flight
constexpr int kBwdLoaders = 2;  // loader waves per workgroup

// Waits until at most n (0..8, wave-uniform) vector-memory operations of this
// wave are outstanding.
__device__ inline void bwd_wait_vm(int n) {
    switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

// The loader waves' side of a stream of T blocks through the ring.  Block s
// goes to slot s % kBwdStages, issued kBwdStages - 1 blocks ahead of its use;
// before barrier s a loader waits only for its copies of block s (the later
// ones may stay in flight, since a wave's copies complete in order).  The
// compute waves take block s between barriers s and s + 1, so the slot that
// block s + kBwdStages - 1 overwrites after barrier s is free.
// issue(s, slot) issues this wave's `own` copies of block s.
template <typename Issue>
__device__ inline void bwd_stream(int T, int own, Issue&& issue) {
    for (int s = 0; s < kBwdStages - 1 && s < T; s++) issue(s, s);
    for (int s = 0; s < T; s++) {
        const int ahead = T - 1 - s < kBwdStages - 2 ? T - 1 - s : kBwdStages - 2;
        bwd_wait_vm(ahead * own);
        bwd_loader_barrier();
        const int nxt = s + kBwdStages - 1;
        if (nxt < T) issue(nxt, nxt % kBwdStages);
    }
}

// 1 KB copies per [32][D] block, and how many of them wave w of nwaves issues
template <int D>
constexpr int block_copies() { return kBwdBlk / (64 / (D / 8)); }
template <int D>
__device__ inline int block_copies_of(int w, int nwaves) {
    return w < block_copies<D>() ? (block_copies<D>() - 1 - w) / nwaves + 1 : 0;
}
constexpr int kBwdKWaves = 8;   // key kernel: at most 8 key tiles at a time
constexpr int kBwdDiag = 16 * 48; // key kernel: floats of one tile's diagonal scratch

// compute waves of the key kernel: 8 for 128-wide heads (one workgroup per
// CU, bounded by LDS), 6 otherwise, so that two workgroups of 8 waves fit a
// CU's registers
__host__ __device__ constexpr int bwd_kv_waves(int head_dim) { return head_dim == 128 ? 8 : 6; }
// the loaders' waits stay within bwd_wait_vm's range
static_assert((kBwdStages - 2) * 2 * ((block_copies<128>() + kBwdLoaders - 1) / kBwdLoaders) <= 8,
              "copies in flight per loader wave");

struct BwdBigLds {
    int NPX;                     // tokens rounded up to a whole block
    size_t tw, kb, qb, bias, dtab, stat, diag, buf, buf_bytes, total_q, total_k;
};

__host__ __device__ inline BwdBigLds bwd_big_lds(const Geometry& g, int kw) {
    BwdBigLds L;
    L.NPX = (g.N + kBwdBlk - 1) / kBwdBlk * kBwdBlk;
    const size_t tab = ((size_t)g.table_size * 4 + 15) / 16 * 16;
    L.tw = 0;                                               // int per token
    L.kb = L.tw + (size_t)L.NPX * 4;                        // int per token: key bias offset
    L.qb = L.kb + (size_t)L.NPX * 4;                        // int per token: query bias offset
    L.bias = L.qb + (size_t)L.NPX * 4;                      // the head's table slice
    L.dtab = L.bias + tab;                                  // key kernel: the unit's share
    L.stat = L.dtab + tab;                                  // key kernel: lse2, D per query
    L.diag = L.stat + (size_t)L.NPX * 8;                    // key kernel: per compute wave 2 x 16 x 48 diagonal scratch
    L.buf = L.diag + (size_t)kw * 2 * kBwdDiag * 4;
    L.buf_bytes = (size_t)kBwdBlk * g.head_dim * 2;         // one [32][D] bf16 block
    L.total_q = L.dtab + 2 * kBwdStages * L.buf_bytes;      // query kernel: the K, V ring from dtab on
    L.total_k = L.buf + 2 * kBwdStages * L.buf_bytes;       // key kernel: the Q, dO ring
    return L;
}

// token word of slot n of window (b, wc): row + 1 | mask field << 28, as the
// single-workgroup kernel; a slot past N gets a field no query has
__device__ inline int big_token_word(const Geometry& g, const int wc[3], int b, int n) {
    if (n >= g.N) return 15 << 28;
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
    return ((is_pad ? -1 : tok) + 1) | ((region | (is_pad ? 8 : 0)) << 28);
}

// key and query bias offsets of slot n (the same in every window)
__device__ inline void big_bias_offsets(const Geometry& g, int n, int& kb, int& qb) {
    if (n < g.N) {
        int l[3];
        local_coords(g, n, l[0], l[1], l[2]);
        kb = (l[0] * g.tdy + l[1]) * g.tdx + l[2];
        qb = kb + g.c0;
    } else {
        kb = 0;
        qb = g.table_size - 1; // qb - kb stays inside the table
    }
}

// token table of a unit for the big-window kernels: tw, key and query bias offsets
__device__ inline void big_token_table(const Geometry& g, const int wc[3], int b, int NPX, int* tw, int* kbo,
                                       int* qbo, int nthreads) {
    for (int n = threadIdx.x; n < NPX; n += nthreads) {
        tw[n] = big_token_word(g, wc, b, n);
        big_bias_offsets(g, n, kbo[n], qbo[n]);
    }
}

__device__ inline void unit_coords(const Geometry& g, uint32_t unit, int& h, int& b, int wc[3], uint32_t& wi) {
    wi = fdiv(g.fd_heads, unit);
    h = (int)(unit - wi * (uint32_t)g.heads);
    b = (int)fdiv(g.fd_nW, wi);
    const uint32_t r = wi - (uint32_t)b * (uint32_t)g.nW;
    const uint32_t r2 = fdiv(g.fd_nwin2, r);
    wc[2] = (int)(r - r2 * (uint32_t)g.nwin[2]);
    wc[0] = (int)fdiv(g.fd_nwin1, r2);
    wc[1] = (int)(r2 - (uint32_t)wc[0] * (uint32_t)g.nwin[1]);
}

// copies one [32][D] block of a tensor (rows from the token table; pad and
// past-N rows read row 0) into LDS, swizzled; the calling waves split the
// 1 KB copies.  Returns the copies this wave issued.
template <int D>
__device__ inline int copy_block(const Geometry& g, const uint16_t* src, int h, const int* tw, int t0,
                                 unsigned char* dst, int wave, int nwaves) {
    constexpr int CH = D / 8, RPC = 64 / CH, NC = kBwdBlk / RPC;
    const int lane = threadIdx.x & 63, m0 = lane / CH;
    int issued = 0;
    for (int c = wave; c < NC; c += nwaves) {
        const int r1 = tw[t0 + c * RPC + m0] & kRowMask;
        const uint64_t off = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + h * D +
                             copy_chunk<D>(c * RPC + m0, lane) * 8;
        __builtin_amdgcn_global_load_lds((const void*)(src + off), (lds_void*)(dst + c * 1024), 16, 0, 0);
        issued++;
    }
    return issued;
}

// With lse (and o, the forward's output) the statistics come from the forward
// pass: lse2 = log2(e) * lse and D = rowsum(dO * O), and K and V stream once.
template <int D, int QW>
__global__ __launch_bounds__((QW + kBwdLoaders) * 64) void attn_bf16_bwd_q_kernel(
    Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ table, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    float* __restrict__ stats, uint32_t work0, uint32_t count, const uint16_t* __restrict__ o,
    const float* __restrict__ lse) {
    constexpr int THREADS = (QW + kBwdLoaders) * 64;
    constexpr int KSTEPS = D / 32, DT = D / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    const BwdBigLds L = bwd_big_lds(g, bwd_kv_waves(g.head_dim));
    const int N = g.N, NPX = L.NPX, NB = NPX / kBwdBlk;
    int* tw = (int*)(smem + L.tw);
    int* kbo = (int*)(smem + L.kb);
    int* qbo = (int*)(smem + L.qb);
    float* bias = (float*)(smem + L.bias);
    unsigned char* ring = smem + L.dtab; // kBwdStages slots of a K block and a V block
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;

    const int QB = (N + QW * 16 - 1) / (QW * 16);
    const uint32_t total = count * (uint32_t)QB; // units work0 .. work0 + count - 1
    const uint32_t work = (uint32_t)xcd_work_index(blockIdx.x, total);
    const uint32_t ul = work / (uint32_t)QB;
    const uint32_t unit = work0 + ul;
    const int qblk = (int)(work - ul * (uint32_t)QB);
    int h, b, wc[3];
    uint32_t wi;
    unit_coords(g, unit, h, b, wc, wi);
    const bool masked_window = window_maybe_masked(g, wc);

    big_token_table(g, wc, b, NPX, tw, kbo, qbo, THREADS);
    for (int i = tid; i < g.table_size; i += THREADS) bias[i] = table[(size_t)h * g.table_size + i];
    __syncthreads();

    const int passes = lse != nullptr ? 1 : 2;
    if (wave >= QW) { // loader waves: K and V blocks, once per pass
        const int li = wave - QW;
        bwd_stream(passes * NB, 2 * block_copies_of<D>(li, kBwdLoaders), [&](int s, int slot) {
            const int j = s < NB ? s : s - NB;
            unsigned char* dst = ring + (size_t)slot * 2 * L.buf_bytes;
            copy_block<D>(g, k, h, tw, j * kBwdBlk, dst, li, kBwdLoaders);
            copy_block<D>(g, v, h, tw, j * kBwdBlk, dst + L.buf_bytes, li, kBwdLoaders);
        });
        return;
    }

    // this lane's query and its B operands (query n, d = 32 ks + 8 grp + 0..7)
    const int n = qblk * QW * 16 + wave * 16 + col;
    const bool in_window = n < N;
    const int qword = in_window ? tw[n] : (15 << 28);
    const unsigned qreg = (unsigned)qword >> 28;
    const int r = (qword & kRowMask) - 1;
    const float qvalid = r >= 0 ? 1.f : 0.f; // pad queries have no output, so no gradient
    const int qb = in_window ? qbo[n] : g.table_size - 1;
    bf16x8 qf[KSTEPS], df[KSTEPS];
    {
        const uint64_t base = (uint64_t)(uint32_t)(r < 0 ? 0 : r) * (uint32_t)g.row + h * D + grp * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(q + base + ks * 32));
            df[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(dout + base + ks * 32));
        }
    }

    // S^T and dP^T of key block j (in ring slot `slot`) for this lane's query:
    // tiles t = 0, 1 (keys 16 t + 4 grp + 0..3); S as logits in log2 units
    auto block_products = [&](int slot, int j, f32x4 (&s)[2], f32x4 (&dp)[2]) __attribute__((always_inline)) {
        const uint16_t* Ks = (const uint16_t*)(ring + (size_t)slot * 2 * L.buf_bytes);
        const uint16_t* Vs = (const uint16_t*)(ring + (size_t)slot * 2 * L.buf_bytes + L.buf_bytes);
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int krow = t * 16 + col;
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) {
                const int kslot = k_slot<D>(krow, ks * 4 + grp) * 8;
                a0 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(Ks + krow * D + kslot)), qf[ks], a0);
                a1 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(Vs + krow * D + kslot)), df[ks], a1);
            }
            s[t] = a0;
            dp[t] = a1;
        }
        // logits in log2 units: (scale * s + bias) * log2(e), -inf where masked.
        // The lane's 4 keys are consecutive: their words come in one 16-byte
        // read each, and every bias read is issued before any is used.
        const int key0 = j * kBwdBlk;
        const bool check = masked_window || key0 + kBwdBlk > N;
        u32x4 kb4[2], tw4[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            kb4[t] = *(const u32x4*)(kbo + key0 + t * 16 + grp * 4);
            tw4[t] = *(const u32x4*)(tw + key0 + t * 16 + grp * 4);
        }
        float bv[2][4];
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) bv[t][i] = bias[qb - (int)kb4[t][i]];
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float lg = fmaf(s[t][i], g.scale, bv[t][i]) * kLog2e;
                s[t][i] = check && (tw4[t][i] >> 28) != qreg ? -INFINITY : lg;
            }
    };

    // ---- pass 1: the softmax statistics and D = rowsum(P * dP) at once.  Per
    // lane, over its keys: the running max m, l = sum 2^(logit - m) and
    // dsum = sum 2^(logit - m) dP, both rescaled when m grows; then across the
    // query's 4 lanes.  D = dsum / l.  Skipped when the forward's statistics
    // are given.
    float m_run = -INFINITY, l_run = 0.f, d_run = 0.f;
    int slot = 0;
    for (int j = 0; j < (passes == 2 ? NB : 0); j++) {
        bwd_compute_barrier(); // block j is in its slot
        f32x4 s[2], dp[2];
        block_products(slot, j, s, dp);
        float bm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) bm = fmaxf(bm, s[t][i]);
        const float mn = fmaxf(m_run, bm);
        if (mn != -INFINITY) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn); // 0 while m_run is -inf
            float la = 0.f, da = 0.f;
#pragma unroll
            for (int t = 0; t < 2; t++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float e = __builtin_amdgcn_exp2f(s[t][i] - mn);
                    la += e;
                    da = fmaf(e, dp[t][i], da);
                }
            l_run = fmaf(l_run, alpha, la);
            d_run = fmaf(d_run, alpha, da);
            m_run = mn;
        }
        slot = slot + 1 == kBwdStages ? 0 : slot + 1;
    }
    float m_all = fmaxf(m_run, __shfl_xor(m_run, 16));
    m_all = fmaxf(m_all, __shfl_xor(m_all, 32));
    const float wgt = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_all);
    float l_all = l_run * wgt, d_all = d_run * wgt;
    l_all += __shfl_xor(l_all, 16);
    l_all += __shfl_xor(l_all, 32);
    d_all += __shfl_xor(d_all, 16);
    d_all += __shfl_xor(d_all, 32);
    // P = qvalid * exp2(logit - lse2); a query with no visible key (pad) gets P = 0
    float lse2 = l_all > 0.f ? m_all + log2f(l_all) : 0.f;
    float pscale = l_all > 0.f ? qvalid : 0.f;
    float dsum = pscale == 0.f ? 0.f : d_all / l_all;
    if (passes == 1) {
        // the forward's statistics: every real query sees itself, so its sum is
        // positive; D over the head slice, this lane's 8 d per step and then
        // across the query's 4 lanes
        float part = 0.f;
        if (r >= 0) {
            const uint64_t base = (uint64_t)(uint32_t)r * (uint32_t)g.row + h * D + grp * 8;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) {
                const bf16x8 of = __builtin_bit_cast(bf16x8, *(const u32x4*)(o + base + ks * 32));
#pragma unroll
                for (int e = 0; e < 8; e++) part = fmaf((float)df[ks][e], (float)of[e], part);
            }
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        lse2 = r >= 0 ? lse[(uint64_t)(uint32_t)r * (uint32_t)g.heads + h] * kLog2e : 0.f;
        pscale = qvalid;
        dsum = r >= 0 ? part : 0.f;
    }
    // statistics per query: lse2 (log2 of the softmax normaliser) and D; a pad
    // query gets lse2 = +inf, so that every P it would take is 0
    if (grp == 0 && in_window) {
        float* st = stats + (size_t)ul * 2 * NPX;
        st[n] = pscale == 0.f ? INFINITY : lse2;
        st[NPX + n] = dsum;
    }

    // ---- pass 2: dS and dQ^T = K^T dS^T (the forward's O^T = V^T P^T with K for V, dS for P)
    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < NB; j++) {
        bwd_compute_barrier();
        f32x4 s[2], dp[2];
        block_products(slot, j, s, dp);
        unsigned pk[2][2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            f32x4 ds;
#pragma unroll
            for (int i = 0; i < 4; i++) ds[i] = pscale * __builtin_amdgcn_exp2f(s[t][i] - lse2) * (dp[t][i] - dsum);
            pk[t][0] = pack_bf16x2(ds[0], ds[1]);
            pk[t][1] = pack_bf16x2(ds[2], ds[3]);
        }
        const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{pk[0][0], pk[0][1], pk[1][0], pk[1][1]});
        const unsigned char* Kb = ring + (size_t)slot * 2 * L.buf_bytes;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            // transposed 4 x 16 reads of K: keys 16 t + 4 grp + 0..3, d = 16 dt + col
            u32x2 part[2];
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int row = t * 16 + grp * 4 + (col >> 2);
                const int d = dt * 16 + (col & 3) * 4;
                part[t] = tr_read(Kb + row * (D * 2) + k_slot<D>(row, d >> 3) * 16 + (d & 7) * 2);
            }
            acc[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}), bop,
                             acc[dt]);
        }
        slot = slot + 1 == kBwdStages ? 0 : slot + 1;
    }
    if (r >= 0) {
        uint16_t* op = dq + (uint64_t)(uint32_t)r * (uint32_t)g.row + h * D + grp * 4;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
            *(u32x2*)(op + dt * 16) = u32x2{pack_bf16x2(acc[dt][0] * g.scale, acc[dt][1] * g.scale),
                                            pack_bf16x2(acc[dt][2] * g.scale, acc[dt][3] * g.scale)};
    }
}

// KW = bwd_kv_waves(D) compute waves, a 16-key tile each.
// RUNS: how a diagonal of a 16 x 16 tile splits into runs of one table entry:
// 0, never (the window width is a multiple of 16); 1, at row starts (width of
// at least 8); 2, wherever the entry changes (any width).
template <int D, int KW, int RUNS>
__global__ __launch_bounds__((KW + kBwdLoaders) * 64)
__attribute__((amdgpu_waves_per_eu(KW == 6 ? 4 : 1))) void attn_bf16_bwd_kv_kernel(
    Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ table, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, const float* __restrict__ stats, float* __restrict__ dtab_units, uint32_t work0,
    uint32_t count) {
    static_assert(KW <= kBwdKWaves, "diagonal scratch per compute wave");
    constexpr int THREADS = (KW + kBwdLoaders) * 64;
    constexpr int KSTEPS = D / 32, DT = D / 16;
    constexpr int DIAG = kBwdDiag; // one tile's scratch: [slot][diagonal + slot]
    extern __shared__ __align__(16) unsigned char smem[];
    const BwdBigLds L = bwd_big_lds(g, KW);
    const int N = g.N, NPX = L.NPX, NB = NPX / kBwdBlk;
    int* tw = (int*)(smem + L.tw);
    int* kbo = (int*)(smem + L.kb);
    int* qbo = (int*)(smem + L.qb);
    float* bias = (float*)(smem + L.bias);
    float* dtab = (float*)(smem + L.dtab);
    float* lse = (float*)(smem + L.stat);
    float* dd = lse + NPX;
    float* diag = (float*)(smem + L.diag);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;

    const uint32_t ul = (uint32_t)xcd_work_index(blockIdx.x, count); // unit work0 + ul
    const uint32_t unit = work0 + ul;
    int h, b, wc[3];
    uint32_t wi;
    unit_coords(g, unit, h, b, wc, wi);
    const bool masked_window = window_maybe_masked(g, wc);

    big_token_table(g, wc, b, NPX, tw, kbo, qbo, THREADS);
    for (int i = tid; i < g.table_size; i += THREADS) {
        bias[i] = table[(size_t)h * g.table_size + i];
        dtab[i] = 0.f;
    }
    {
        const float* st = stats + (size_t)ul * 2 * NPX;
        for (int i = tid; i < NPX; i += THREADS) {
            lse[i] = i < N ? st[i] : INFINITY; // slots past N: P = 0
            dd[i] = i < N ? st[NPX + i] : 0.f;
        }
    }
    // the diagonal scratch starts at zero: slots off a tile's diagonals are never written
    for (int i = tid; i < KW * 2 * DIAG; i += THREADS) diag[i] = 0.f;
    __syncthreads();

    unsigned char* ring = smem + L.buf; // kBwdStages slots of a Q block and a dO block
    const int KT = NPX / 16;            // key tiles; the compute waves take them KW at a time
    const int G = (KT + KW - 1) / KW;
    if (wave >= KW) { // loader waves: every Q and dO block, once per group of key tiles
        const int li = wave - KW;
        bwd_stream(G * NB, 2 * block_copies_of<D>(li, kBwdLoaders), [&](int s, int slot) {
            const int j = s - (s / NB) * NB;
            unsigned char* dst = ring + (size_t)slot * 2 * L.buf_bytes;
            copy_block<D>(g, q, h, tw, j * kBwdBlk, dst, li, kBwdLoaders);
            copy_block<D>(g, dout, h, tw, j * kBwdBlk, dst + L.buf_bytes, li, kBwdLoaders);
        });
        bwd_loader_barrier(); // final: the table share is complete
    } else {
        // transposed 4 x 16 read of a [32][D] block: rows t0 + 4 grp + 0..3, d = 16 dt + col
        auto tr_blk = [&](const unsigned char* base, int t0, int dt) __attribute__((always_inline)) {
            const int row = t0 + grp * 4 + (col >> 2);
            const int d = dt * 16 + (col & 3) * 4;
            return tr_read(base + row * (D * 2) + k_slot<D>(row, d >> 3) * 16 + (d & 7) * 2);
        };
        float* sc = diag + wave * 2 * DIAG;     // [tile][slot][diagonal + slot]
        const int dl = lane & 31, tt = lane >> 5; // the diagonal and the tile this lane sums

        int slot = 0;
        for (int kt0 = 0; kt0 < KT; kt0 += KW) {
            const int kt = kt0 + wave;
            const bool active = kt < KT;
            const int m0 = (active ? kt : 0) * 16;
            const int m = m0 + col;
            const int kword = active ? tw[m] : (15 << 28);
            const unsigned kreg = (unsigned)kword >> 28;
            const int kr = (kword & kRowMask) - 1;
            const int kbm = active ? kbo[m] : 0;
            const bool key_in = active && m < N; // slots past N see no query: masked in every block
            // B operands: key m, d = 32 ks + 8 grp + 0..7 (pad keys read row 0; they are masked)
            bf16x8 kf[KSTEPS], vf[KSTEPS];
            {
                const uint64_t base = (uint64_t)(uint32_t)(kr < 0 ? 0 : kr) * (uint32_t)g.row + h * D + grp * 8;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ks++) {
                    kf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(k + base + ks * 32));
                    vf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(v + base + ks * 32));
                }
            }
            f32x4 av[DT], ak[DT]; // dV^T and dK^T: lane (key m, d = 16 dt + 4 grp + 0..3)
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                av[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
                ak[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            for (int j = 0; j < NB; j++) {
                bwd_compute_barrier(); // query block j is in its slot
                if (active) {
                    const unsigned char* Qb = ring + (size_t)slot * 2 * L.buf_bytes;
                    const unsigned char* Ob = Qb + L.buf_bytes;
                    const uint16_t* Qs = (const uint16_t*)Qb;
                    const uint16_t* dOs = (const uint16_t*)Ob;
                    const int nb = j * kBwdBlk;
                    // S = Q K^T and dP = dO V^T: lane (key m, queries 16 t + 4 grp + 0..3 of the block)
                    f32x4 sv[2], dpv[2];
#pragma unroll
                    for (int t = 0; t < 2; t++) {
                        const int qrow = t * 16 + col;
                        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KSTEPS; ks++) {
                            const int ksl = k_slot<D>(qrow, ks * 4 + grp) * 8;
                            a0 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(Qs + qrow * D + ksl)), kf[ks], a0);
                            a1 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(dOs + qrow * D + ksl)), vf[ks], a1);
                        }
                        sv[t] = a0;
                        dpv[t] = a1;
                    }
                    const bool check = masked_window || nb + kBwdBlk > N;
                    unsigned pp[2][2], ps[2][2];
                    // the lane's key is fixed: one past N is masked whatever the query block
#pragma unroll
                    for (int t = 0; t < 2; t++) {
                        // the words of the lane's 4 queries (consecutive: one 16-byte read
                        // each), then every bias read before any is used
                        const int n4 = nb + t * 16 + grp * 4;
                        const u32x4 qb4 = *(const u32x4*)(qbo + n4);
                        const f32x4 ls4 = *(const f32x4*)(lse + n4);
                        float lg[4];
#pragma unroll
                        for (int i = 0; i < 4; i++) lg[i] = bias[(int)qb4[i] - kbm];
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            lg[i] = key_in ? fmaf(sv[t][i], g.scale, lg[i]) * kLog2e : -INFINITY;
                        if (check) { // wave-uniform: queries of another region, pad or past N
                            const u32x4 tw4 = *(const u32x4*)(tw + n4);
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                if ((tw4[i] >> 28) != kreg) lg[i] = -INFINITY;
                        }
                        const f32x4 dd4 = *(const f32x4*)(dd + n4);
                        f32x4 p, ds;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            p[i] = __builtin_amdgcn_exp2f(lg[i] - ls4[i]);
                            ds[i] = p[i] * (dpv[t][i] - dd4[i]);
                        }
                        pp[t][0] = pack_bf16x2(p[0], p[1]);
                        pp[t][1] = pack_bf16x2(p[2], p[3]);
                        ps[t][0] = pack_bf16x2(ds[0], ds[1]);
                        ps[t][1] = pack_bf16x2(ds[2], ds[3]);
                        // pair (query a = 4 grp + i, key col) of tile t lies on diagonal
                        // d = a - col + 15 (0..30); its term goes to [t][a][d + a], rows
                        // of 48: word 50 a - col + 15, which spreads a write's 64 lanes
                        // evenly over the 32 banks
#pragma unroll
                        for (int i = 0; i < 4; i++) sc[t * DIAG + 50 * (4 * grp + i) - col + 15] = ds[i];
                    }
                    // The block's dS into the unit's table share.  Along a diagonal of a
                    // 16 x 16 tile the table entry changes only where the query or the
                    // key crosses a window row, so lane (tt, dl) sums diagonal dl - 15 of
                    // tile tt (slots off the diagonal hold 0) and adds each run of equal
                    // entries with one atomic: a single run when the window width is a
                    // multiple of 16, a few otherwise.
                    if (m0 < N) { // wave-uniform; terms past N are 0
                        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): this wave's terms landed
                        const int n0 = nb + tt * 16, dgl = dl - 15;
                        if (dl < 31 && n0 < N) {
                            // slot a of this diagonal pairs query n0 + a with key m0 + a - dgl
                            const float* sd = sc + tt * DIAG;
                            if (RUNS == 0) {
                                float x[16];
#pragma unroll
                                for (int a = 0; a < 16; a++) x[a] = sd[49 * a + dl];
                                float run = 0.f;
#pragma unroll
                                for (int a = 0; a < 16; a++) run += x[a];
                                atomicAdd(&dtab[qbo[n0] - kbo[m0] + dgl], run);
                            } else if (RUNS == 1) {
                                // A window row holds at least 8 tokens, so at most two row
                                // starts of the queries and two of the keys fall strictly
                                // inside the diagonal: they cut it into at most five runs
                                // of one entry each.  The prefix sums of the diagonal go
                                // back into its own slots (the others stay 0); a run's sum
                                // is the difference of the prefix sums at its ends, its
                                // entry the table words at its first slot.
                                float* sdw = sc + tt * DIAG;
                                const int alo = dgl > 0 ? dgl : 0, ahi = dgl < 0 ? 16 + dgl : 16;
                                float pre = 0.f;
#pragma unroll
                                for (int half = 0; half < 2; half++) {
                                    float x[8];
#pragma unroll
                                    for (int c = 0; c < 8; c++) x[c] = sd[49 * (8 * half + c) + dl];
#pragma unroll
                                    for (int c = 0; c < 8; c++) {
                                        const int a = 8 * half + c;
                                        if (a >= alo && a < ahi) sdw[49 * a + dl] = pre;
                                        pre += x[c];
                                    }
                                }
                                // row starts inside (alo, ahi): the query n0 + a or the key
                                // m0 + a - dgl at a multiple of the window width
                                const int w2 = g.win[2];
                                const int rq = n0 % w2, rk = ((m0 - dgl) % w2 + w2) % w2;
                                int c[4];
                                c[0] = rq == 0 ? w2 : w2 - rq;
                                c[1] = c[0] + w2;
                                c[2] = rk == 0 ? w2 : w2 - rk;
                                c[3] = c[2] + w2;
#pragma unroll
                                for (int i = 0; i < 4; i++) c[i] = c[i] > alo && c[i] < ahi ? c[i] : ahi;
                                auto order = [&](int i, int j) __attribute__((always_inline)) {
                                    const int lo = min(c[i], c[j]), hi = max(c[i], c[j]);
                                    c[i] = lo;
                                    c[j] = hi;
                                };
                                order(0, 1);
                                order(2, 3);
                                order(0, 2);
                                order(1, 3);
                                order(1, 2);
                                float pc[4];
#pragma unroll
                                for (int i = 0; i < 4; i++) pc[i] = c[i] < ahi ? sd[49 * c[i] + dl] : pre;
                                const int st[5] = {alo, c[0], c[1], c[2], c[3]};
                                const int en[5] = {c[0], c[1], c[2], c[3], ahi};
                                const float sum[5] = {pc[0], pc[1] - pc[0], pc[2] - pc[1], pc[3] - pc[2], pre - pc[3]};
#pragma unroll
                                for (int r = 0; r < 5; r++)
                                    if (st[r] < en[r])
                                        atomicAdd(&dtab[qbo[n0 + st[r]] - kbo[m0 + st[r] - dgl]], sum[r]);
                            } else {
                                float run = 0.f;
                                int ecur = -1;
#pragma unroll
                                for (int half = 0; half < 2; half++) {
                                    float x[8];
#pragma unroll
                                    for (int c = 0; c < 8; c++) x[c] = sd[49 * (8 * half + c) + dl];
#pragma unroll
                                    for (int c = 0; c < 8; c++) {
                                        const int a = 8 * half + c;
                                        if (a - dgl >= 0 && a - dgl < 16) {
                                            const int ea = qbo[n0 + a] - kbo[m0 + a - dgl];
                                            if (ea != ecur) {
                                                if (ecur >= 0) atomicAdd(&dtab[ecur], run);
                                                ecur = ea;
                                                run = 0.f;
                                            }
                                            run += x[c];
                                        }
                                    }
                                }
                                if (ecur >= 0) atomicAdd(&dtab[ecur], run);
                            }
                        }
                        __builtin_amdgcn_s_waitcnt(0xC07F); // the reads are done before the next block's terms
                    }
                    const bf16x8 bp = __builtin_bit_cast(bf16x8, u32x4{pp[0][0], pp[0][1], pp[1][0], pp[1][1]});
                    const bf16x8 bs = __builtin_bit_cast(bf16x8, u32x4{ps[0][0], ps[0][1], ps[1][0], ps[1][1]});
                    // dV^T += dO^T P and dK^T += Q^T dS, contracting over the block's 32 queries
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const u32x2 o0 = tr_blk(Ob, 0, dt), o1 = tr_blk(Ob, 16, dt);
                        const u32x2 q0 = tr_blk(Qb, 0, dt), q1 = tr_blk(Qb, 16, dt);
                        av[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{o0[0], o0[1], o1[0], o1[1]}), bp, av[dt]);
                        ak[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]}), bs, ak[dt]);
                    }
                }
                slot = slot + 1 == kBwdStages ? 0 : slot + 1;
            }
            if (active && kr >= 0) {
                const uint64_t base = (uint64_t)(uint32_t)kr * (uint32_t)g.row + h * D + grp * 4;
#pragma unroll
                for (int dt = 0; dt < DT; dt++) {
                    *(u32x2*)(dv + base + dt * 16) =
                        u32x2{pack_bf16x2(av[dt][0], av[dt][1]), pack_bf16x2(av[dt][2], av[dt][3])};
                    *(u32x2*)(dk + base + dt * 16) = u32x2{pack_bf16x2(ak[dt][0] * g.scale, ak[dt][1] * g.scale),
                                                           pack_bf16x2(ak[dt][2] * g.scale, ak[dt][3] * g.scale)};
                }
            }
        }
        bwd_compute_barrier(); // final: every atomic of the table share has landed
    }
    float* dst = dtab_units + (size_t)ul * g.table_size;
    for (int e = tid; e < g.table_size; e += THREADS) dst[e] = dtab[e];
}

// ---- attn_bf16_bwd_kvp_kernel: the key kernel with the table gradient summed
// over windows before it is summed over offsets.
//
// A table entry depends only on the window-local positions of its query and
// key, so dtable[e] = sum, over the local pairs (n, m) of entry e, of
// S[n][m] = sum over windows of dS[n][m].  A workgroup takes one head, one
// group of kKvpTiles key tiles and a run of consecutive windows.  Each of its
// compute waves owns a key tile and one 16-query half of every 32-query
// block, and adds each window's dS of its pairs into registers: one add per
// term, where attn_bf16_bwd_kv_kernel parks the terms in LDS and adds runs of
// each tile diagonal with atomics.  At the end every wave writes its pair
// sums; pair_runs_kernel adds the runs of windows in order and
// dtable_pairs_kernel sums each entry's pairs in query order, so this table
// gradient is bitwise reproducible.
//
// The two halves of a key tile each hold a share of its dK and dV; at the end
// of a window the second half leaves its share in LDS and the first adds it
// after the next barrier and stores both.  Four loader waves stream the Q
// and dO blocks of the current window through the ring, two or three blocks
// per step (one barrier per step), and, from the start of a window on, build
// the next window's token words and copy its statistics, K and V (the
// group's keys) into the other of two window buffers; the compute waves take
// their key tile's K and V fragments into registers at the window's start.
// Eight compute waves (4 key tiles) keep the workgroup at about 160 VGPRs, 3 waves
// per SIMD; 12 (6 key tiles) need more than the 128 of 4 waves per SIMD and
// spill.
constexpr int kKvpTiles = 4;                              // key tiles per group
constexpr int kKvpWaves = 2 * kKvpTiles;                  // compute waves: (key tile, query half)
constexpr int kKvpLoaders = 4;
constexpr int kKvpBlocks = 9;                             // 32-query blocks per window, at most
constexpr int kKvpWorkgroups = 256;                       // aimed at: one per compute unit
constexpr int kKvpSums = kKvpWaves * kKvpBlocks * 4 * 64; // pair sums per workgroup (floats)

// blocks per step: three where a window has at least 7 blocks (3 steps or
// more, which the loaders' token words need), else two
__host__ __device__ constexpr int kvp_step_blocks(int nb) { return nb >= 7 ? 3 : 2; }

struct KvpLds {
    int NPX;
    size_t kbo, qbo, bias, win, win_bytes, tw, stat, kt, vt, ring, buf_bytes, exch, total;
};

__host__ __device__ inline KvpLds kvp_lds(const Geometry& g) {
    KvpLds L;
    const size_t D = (size_t)g.head_dim;
    L.NPX = (g.N + kBwdBlk - 1) / kBwdBlk * kBwdBlk;
    L.kbo = 0;                                                  // int per slot: key bias offset
    L.qbo = L.kbo + (size_t)L.NPX * 4;                          // int per slot: query bias offset
    L.bias = L.qbo + (size_t)L.NPX * 4;                         // the head's table slice
    L.win = L.bias + ((size_t)g.table_size * 4 + 15) / 16 * 16; // two window buffers
    L.tw = 0;                                                   // per window: token words,
    L.stat = L.tw + (size_t)L.NPX * 4;                          //   lse2 and D per query,
    L.kt = L.stat + (size_t)L.NPX * 8;                          //   K and V of the group's keys
    L.vt = L.kt + (size_t)kKvpTiles * 16 * D * 2;
    L.win_bytes = L.vt + (size_t)kKvpTiles * 16 * D * 2;
    L.ring = L.win + 2 * L.win_bytes;                           // kBwdStages slots of a step: two
    L.buf_bytes = (size_t)kBwdBlk * D * 2;                      //   or three blocks of Q and dO each
    L.exch = L.ring + 2 * kvp_step_blocks(L.NPX / kBwdBlk) * kBwdStages * L.buf_bytes;
                                                                // per key tile: the second half's dV, dK
    L.total = L.exch + (size_t)kKvpTiles * 2 * (D / 16) * 64 * 16;
    return L;
}

// Waits until at most n (wave-uniform) vector-memory operations of this wave
// are outstanding; past 15 it waits for all of them.
__device__ inline void bwd_wait_vm_n(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(vmcnt_imm(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(vmcnt_imm(14)); break;
    case 15: __builtin_amdgcn_s_waitcnt(vmcnt_imm(15)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

// global window index -> batch item and window coordinates
__device__ inline void window_of(const Geometry& g, uint32_t wi, int& b, int wc[3]) {
    b = (int)fdiv(g.fd_nW, wi);
    const uint32_t r = wi - (uint32_t)b * (uint32_t)g.nW;
    const uint32_t r2 = fdiv(g.fd_nwin2, r);
    wc[2] = (int)(r - r2 * (uint32_t)g.nwin[2]);
    wc[0] = (int)fdiv(g.fd_nwin1, r2);
    wc[1] = (int)(r2 - (uint32_t)wc[0] * (uint32_t)g.nwin[1]);
}

// copy_block with each lane's source row computed from the window instead of
// read from a token table in LDS
template <int D>
__device__ inline int copy_block_rows(const Geometry& g, const uint16_t* src, int h, const int wc[3], int b, int t0,
                                      unsigned char* dst, int wave, int nwaves) {
    constexpr int CH = D / 8, RPC = 64 / CH, NC = kBwdBlk / RPC;
    const int lane = threadIdx.x & 63, m0 = lane / CH;
    int issued = 0;
    for (int c = wave; c < NC; c += nwaves) {
        const int r1 = big_token_word(g, wc, b, t0 + c * RPC + m0) & kRowMask;
        const uint64_t off = (uint64_t)(uint32_t)(r1 == 0 ? 0 : r1 - 1) * (uint32_t)g.row + h * D +
                             copy_chunk<D>(c * RPC + m0, lane) * 8;
        __builtin_amdgcn_global_load_lds((const void*)(src + off), (lds_void*)(dst + c * 1024), 16, 0, 0);
        issued++;
    }
    return issued;
}

// Workgroup wg of heads * runs * groups (run of windows, key group), over
// windows w0 .. w0 + nw - 1 (the units whose statistics are at
// stats[((w - w0) * heads + h) * 2 NPX]); pair sums to sums[wg * kKvpSums].
template <int D, int SB>
__global__ __launch_bounds__((kKvpWaves + kKvpLoaders) * 64) void attn_bf16_bwd_kvp_kernel(
    Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ table, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, const float* __restrict__ stats, float* __restrict__ sums, uint32_t w0, uint32_t nw,
    int runs, int groups) {
    constexpr int THREADS = (kKvpWaves + kKvpLoaders) * 64;
    constexpr int KSTEPS = D / 32, DT = D / 16;
    static_assert(kKvpTiles * 16 % kBwdBlk == 0, "a group's keys copy as whole blocks");
    extern __shared__ __align__(16) unsigned char smem[];
    const KvpLds L = kvp_lds(g);
    const int N = g.N, NPX = L.NPX, NB = NPX / kBwdBlk;
    int* kbo = (int*)(smem + L.kbo);
    int* qbo = (int*)(smem + L.qbo);
    float* bias = (float*)(smem + L.bias);
    unsigned char* ring = smem + L.ring;
    f32x4* exch = (f32x4*)(smem + L.exch);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;

    // workgroup -> (head, run, key group): the groups of a run are neighbours
    // on one XCD, so the Q and dO blocks that each of them streams share its L2
    const int wg = (int)xcd_work_index(blockIdx.x, (int64_t)g.heads * runs * groups);
    const int kg = wg % groups;
    const int run = (wg / groups) % runs;
    const int h = wg / (groups * runs);
    const uint32_t wbeg = w0 + (uint32_t)((uint64_t)nw * run / runs);
    const int nwin = (int)(w0 + (uint32_t)((uint64_t)nw * (run + 1) / runs) - wbeg);

    for (int n = tid; n < NPX; n += THREADS) big_bias_offsets(g, n, kbo[n], qbo[n]);
    for (int i = tid; i < g.table_size; i += THREADS) bias[i] = table[(size_t)h * g.table_size + i];
    if (nwin > 0) {
        int b, wc[3];
        window_of(g, wbeg, b, wc);
        int* tw0 = (int*)(smem + L.win + L.tw);
        for (int n = tid; n < NPX; n += THREADS) tw0[n] = big_token_word(g, wc, b, n);
    }
    __syncthreads();

    // A step takes SB 32-query blocks of a window (the last step the rest);
    // every window's NS steps stream through the ring.
    const int NS = (NB + SB - 1) / SB, T = nwin * NS;
    if (wave >= kKvpWaves) {
        const int li = wave - kKvpWaves;
        const int per_block = 2 * block_copies_of<D>(li, kKvpLoaders); // this loader's copies per block
        auto own = [&](int s) __attribute__((always_inline)) {         // ... per step s
            const int js = s % NS;
            return (NB - SB * js < SB ? NB - SB * js : SB) * per_block;
        };
        // window i's token words (unless written already), K and V of the
        // group's keys, and its statistics, into window buffer i & 1; returns
        // the copies issued
        auto prologue = [&](int i, bool words) __attribute__((always_inline)) {
            int b, wc[3];
            window_of(g, wbeg + i, b, wc);
            unsigned char* wb = smem + L.win + (size_t)(i & 1) * L.win_bytes;
            if (words) {
                int* tw = (int*)(wb + L.tw);
                for (int n = li * 64 + lane; n < NPX; n += kKvpLoaders * 64) tw[n] = big_token_word(g, wc, b, n);
            }
            int issued = 0;
            for (int c = 0; c < kKvpTiles * 16 / kBwdBlk; c++) {
                const int t0 = kg * kKvpTiles * 16 + c * kBwdBlk;
                issued += copy_block_rows<D>(g, k, h, wc, b, t0, wb + L.kt + c * L.buf_bytes, li, kKvpLoaders);
                issued += copy_block_rows<D>(g, v, h, wc, b, t0, wb + L.vt + c * L.buf_bytes, li, kKvpLoaders);
            }
            // lse2 and D: 2 NPX floats, 16 bytes per lane (lane 0 of every copy is in range)
            const float* st = stats + ((size_t)(wbeg + i - w0) * g.heads + h) * 2 * NPX;
            const int bytes = NPX * 8;
            for (int c = li; c * 1024 < bytes; c += kKvpLoaders) {
                if (c * 1024 + lane * 16 < bytes)
                    __builtin_amdgcn_global_load_lds((const void*)(st + c * 256 + lane * 4),
                                                     (lds_void*)(wb + L.stat + c * 1024), 16, 0, 0);
                issued++;
            }
            return issued;
        };
        auto issue_step = [&](int s) __attribute__((always_inline)) {
            const int i = s / NS, js = s - i * NS;
            const int* tw = (const int*)(smem + L.win + (size_t)(i & 1) * L.win_bytes + L.tw);
            unsigned char* dst = ring + (size_t)(s % kBwdStages) * 2 * SB * L.buf_bytes;
            for (int u = 0; u < SB && SB * js + u < NB; u++) {
                const int j = SB * js + u;
                copy_block<D>(g, q, h, tw, j * kBwdBlk, dst + u * 2 * L.buf_bytes, li, kKvpLoaders);
                copy_block<D>(g, dout, h, tw, j * kBwdBlk, dst + (u * 2 + 1) * L.buf_bytes, li, kKvpLoaders);
            }
        };
        // Issue order: window 0's prologue, steps 0 and 1; after barrier s,
        // the next window's prologue when s starts a window, then step s + 2.
        // Before barrier s a loader waits for its copies of step s; the ones
        // issued after them are step s + 1 and the prologue of step s - 1.
        // Window i + 1's first steps are issued at steps (i + 1) NS - 2 and
        // - 1, after the barrier that follows the prologue writing its token
        // words (NS >= 3).
        if (nwin > 0) prologue(0, false);
        for (int s = 0; s < kBwdStages - 1 && s < T; s++) issue_step(s);
        int pro = 0; // prologue copies issued at the previous step
        for (int s = 0; s < T; s++) {
            bwd_wait_vm_n(pro + (s + 1 < T ? own(s + 1) : 0));
            bwd_loader_barrier();
            const int i = s / NS;
            pro = (s == i * NS && i + 1 < nwin) ? prologue(i + 1, true) : 0;
            if (s + kBwdStages - 1 < T) issue_step(s + kBwdStages - 1);
        }
        bwd_loader_barrier(); // final: the last window's dV and dK shares
        return;
    }

    // compute wave: key tile kg * kKvpTiles + kk, queries 16 th .. 16 th + 15 of each block
    const int kk = wave >> 1, th = wave & 1;
    const int m = (kg * kKvpTiles + kk) * 16 + col; // the lane's key slot
    const bool active = (kg * kKvpTiles + kk) * 16 < NPX;
    const bool key_in = active && m < N; // slots past N are masked in every block
    const int kbm = key_in ? kbo[m] : 0;
    const int krow = kk * 16 + col;      // its row in the window buffer's K and V
    // transposed 4 x 16 read of a [32][D] block: rows t0 + 4 grp + 0..3, d = 16 dt + col
    auto tr_blk = [&](const unsigned char* base, int t0, int dt) __attribute__((always_inline)) {
        const int row = t0 + grp * 4 + (col >> 2);
        const int d = dt * 16 + (col & 3) * 4;
        return tr_read(base + row * (D * 2) + k_slot<D>(row, d >> 3) * 16 + (d & 7) * 2);
    };
    f32x4* ex = exch + (size_t)kk * 2 * DT * 64;
    f32x4 acc[kKvpBlocks]; // pair sums: block j, queries 32 j + 16 th + 4 grp + 0..3, key m
#pragma unroll
    for (int j = 0; j < kKvpBlocks; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 av[DT], ak[DT]; // dV^T and dK^T shares: lane (key m, d = 16 dt + 4 grp + 0..3)
    // the first half adds the second's share and stores the key tile's dV, dK
    auto finish = [&](int kr) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            av[dt] += ex[dt * 64 + lane];
            ak[dt] += ex[(DT + dt) * 64 + lane];
        }
        if (kr >= 0) {
            const uint64_t base = (uint64_t)(uint32_t)kr * (uint32_t)g.row + h * D + grp * 4;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                *(u32x2*)(dv + base + dt * 16) =
                    u32x2{pack_bf16x2(av[dt][0], av[dt][1]), pack_bf16x2(av[dt][2], av[dt][3])};
                *(u32x2*)(dk + base + dt * 16) = u32x2{pack_bf16x2(ak[dt][0] * g.scale, ak[dt][1] * g.scale),
                                                       pack_bf16x2(ak[dt][2] * g.scale, ak[dt][3] * g.scale)};
            }
        }
    };
    int slot = 0, kr = -1;
    bf16x8 kf[KSTEPS], vf[KSTEPS]; // B operands of the key tile: key m, d = 32 ks + 8 grp + 0..7
    for (int i = 0; i < nwin; i++) {
        const unsigned char* wb = smem + L.win + (size_t)(i & 1) * L.win_bytes;
        const int* tw = (const int*)(wb + L.tw);
        const float* lse = (const float*)(wb + L.stat);
        const float* dd = lse + NPX;
        const uint16_t* Kt = (const uint16_t*)(wb + L.kt);
        const uint16_t* Vt = (const uint16_t*)(wb + L.vt);
        int b, wc[3];
        window_of(g, wbeg + i, b, wc);
        const bool masked_window = window_maybe_masked(g, wc);
        unsigned kreg = 15;
        for (int js = 0; js < NS; js++) {
            {
                bwd_compute_barrier(); // step js of window i is in its slot
                if (js == 0) {
                    if (th == 0 && active && i > 0) finish(kr); // the previous window's key tile
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        av[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        ak[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                    const int kword = active ? tw[m] : (15 << 28);
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ks++) {
                        const int kc = k_slot<D>(krow, ks * 4 + grp) * 8;
                        kf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Kt + krow * D + kc));
                        vf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Vt + krow * D + kc));
                    }
                    kreg = (unsigned)kword >> 28;
                    kr = (kword & kRowMask) - 1;
                }
#pragma unroll
                for (int u = 0; u < SB; u++) {
                    const int j = SB * js + u;
                    if (!active || j >= NB) continue;
                    const unsigned char* Qb = ring + (size_t)slot * 2 * SB * L.buf_bytes + u * 2 * L.buf_bytes;
                    const unsigned char* Ob = Qb + L.buf_bytes;
                    const uint16_t* Qs = (const uint16_t*)Qb;
                    const uint16_t* dOs = (const uint16_t*)Ob;
                    const int nb = j * kBwdBlk, qrow = th * 16 + col;
                    // S = Q K^T and dP = dO V^T: lane (key m, queries nb + 16 th + 4 grp + 0..3)
                    f32x4 s4 = {0.f, 0.f, 0.f, 0.f}, dp4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ks++) {
                        const int qc = k_slot<D>(qrow, ks * 4 + grp) * 8;
                        s4 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(Qs + qrow * D + qc)), kf[ks], s4);
                        dp4 = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)(dOs + qrow * D + qc)), vf[ks], dp4);
                    }
                    const int n4 = nb + th * 16 + grp * 4;
                    const u32x4 qb4 = *(const u32x4*)(qbo + n4);
                    const f32x4 ls4 = *(const f32x4*)(lse + n4);
                    const f32x4 dd4 = *(const f32x4*)(dd + n4);
                    float lg[4];
#pragma unroll
                    for (int ii = 0; ii < 4; ii++) lg[ii] = bias[(int)qb4[ii] - kbm];
                    f32x4 p, ds;
#pragma unroll
                    for (int ii = 0; ii < 4; ii++) {
                        const float x = key_in ? fmaf(s4[ii], g.scale, lg[ii]) * kLog2e : -INFINITY;
                        p[ii] = __builtin_amdgcn_exp2f(x - ls4[ii]);
                        ds[ii] = p[ii] * (dp4[ii] - dd4[ii]);
                    }
                    if (masked_window || nb + kBwdBlk > N) { // wave-uniform
                        // queries of another region, pad queries, and slots past N (whose
                        // statistics are not written) take no weight
                        const u32x4 tw4 = *(const u32x4*)(tw + n4);
#pragma unroll
                        for (int ii = 0; ii < 4; ii++) {
                            const bool vis = key_in && (tw4[ii] >> 28) == kreg;
                            p[ii] = vis ? p[ii] : 0.f;
                            ds[ii] = vis ? ds[ii] : 0.f;
                        }
                    }
                    // acc[j] += ds, with j a register index (the loop is not unrolled)
                    switch (j) {
                    case 0: acc[0] += ds; break;
                    case 1: acc[1] += ds; break;
                    case 2: acc[2] += ds; break;
                    case 3: acc[3] += ds; break;
                    case 4: acc[4] += ds; break;
                    case 5: acc[5] += ds; break;
                    case 6: acc[6] += ds; break;
                    case 7: acc[7] += ds; break;
                    default: acc[8] += ds; break;
                    }
                    const bf16x8 bp = __builtin_bit_cast(
                        bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), 0u, 0u});
                    const bf16x8 bs = __builtin_bit_cast(
                        bf16x8, u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), 0u, 0u});
                    // dV^T += dO^T P and dK^T += Q^T dS over this half's 16 queries (the
                    // 32-deep product with its other half zero: one opcode per chain)
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const u32x2 o = tr_blk(Ob, th * 16, dt), qq = tr_blk(Qb, th * 16, dt);
                        av[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{o[0], o[1], 0u, 0u}), bp, av[dt]);
                        ak[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{qq[0], qq[1], 0u, 0u}), bs, ak[dt]);
                    }
                }
                slot = slot + 1 == kBwdStages ? 0 : slot + 1;
                if (js == NS - 1 && th == 1 && active) { // this half's share for the first half
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        ex[dt * 64 + lane] = av[dt];
                        ex[(DT + dt) * 64 + lane] = ak[dt];
                    }
                }
            }
        }
    }
    bwd_compute_barrier(); // final: the last window's second-half shares
    if (th == 0 && active && nwin > 0) finish(kr);
    float* dst = sums + (size_t)wg * kKvpSums + (size_t)wave * kKvpBlocks * 4 * 64;
#pragma unroll
    for (int j = 0; j < kKvpBlocks; j++)
#pragma unroll
        for (int ii = 0; ii < 4; ii++) dst[(j * 4 + ii) * 64 + lane] = acc[j][ii];
}

// pairs[(h * groups + kg) * kKvpSums + x] = sum over runs r, in order, of the
// workgroup sums of (h, r, kg)
__global__ __launch_bounds__(256) void pair_runs_kernel(int heads, int runs, int groups, const float* __restrict__ sums,
                                                        float* __restrict__ pairs) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)heads * groups * kKvpSums) return;
    const int x = (int)(idx % kKvpSums), hg = (int)(idx / kKvpSums);
    const int h = hg / groups, kg = hg - h * groups;
    float acc = 0.f;
    for (int r = 0; r < runs; r++) acc += sums[((size_t)(h * runs + r) * groups + kg) * kKvpSums + x];
    pairs[idx] = acc;
}

// dtable[e][h] = (accumulate ? dtable[e][h] : 0) + the sum of the pair sums
// of (n, m), m the key at offset e from query n (entry e = ((dt + w_t - 1) tdy
// + dy + w_y - 1) tdx + dx + w_x - 1 for the local offset (dt, dy, dx) = query
// - key).  A wave per entry: lane l adds queries l, l + 64, ... in order, then
// the lanes' sums are added in a fixed butterfly order.
__global__ __launch_bounds__(256) void dtable_pairs_kernel(Geometry g, int groups, const float* __restrict__ pairs,
                                                           float* __restrict__ dtable, int accumulate) {
    const int idx = blockIdx.x * 4 + (threadIdx.x >> 6); // h * ts + e
    const int lane = threadIdx.x & 63;
    if (idx >= g.heads * g.table_size) return; // wave-uniform
    const int h = idx / g.table_size, e = idx - h * g.table_size;
    const int ex = e % g.tdx, r = e / g.tdx;
    const int oy = r % g.tdy - (g.win[1] - 1), ot = r / g.tdy - (g.win[0] - 1), ox = ex - (g.win[2] - 1);
    const float* ph = pairs + (size_t)h * groups * kKvpSums;
    float acc = 0.f;
    for (int n = lane; n < g.N; n += 64) {
        int lt, ly, lx;
        local_coords(g, n, lt, ly, lx);
        const int mt = lt - ot, my = ly - oy, mx = lx - ox;
        if (mt < 0 || mt >= g.win[0] || my < 0 || my >= g.win[1] || mx < 0 || mx >= g.win[2]) continue;
        const int m = (mt * g.win[1] + my) * g.win[2] + mx;
        const int kg = (m >> 4) / kKvpTiles, kk = (m >> 4) - kg * kKvpTiles;
        const int wave = 2 * kk + ((n >> 4) & 1), l = ((n >> 2) & 3) * 16 + (m & 15);
        acc += ph[(size_t)kg * kKvpSums + ((size_t)(wave * kKvpBlocks + (n >> 5)) * 4 + (n & 3)) * 64 + l];
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) acc += __shfl_xor(acc, sh);
    if (lane == 0) {
        const size_t o = (size_t)e * g.heads + h;
        dtable[o] = (accumulate ? dtable[o] : 0.f) + acc;
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
    float* __restrict__ dv, float* __restrict__ dtab_units, uint32_t work0, uint32_t count) {
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

    const int64_t work = (int64_t)work0 + xcd_work_index(blockIdx.x, count);
    const int64_t wi = work / g.heads;
    const int h = (int)(work - wi * g.heads);

    fill_token_tables(g, wi, false, N, kword, qword, rowi);
    for (int i = threadIdx.x; i < g.table_size; i += blockDim.x) bias[i] = table[(int64_t)h * g.table_size + i];
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
    float* dst = dtab_units + (size_t)(work - work0) * g.table_size;
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

// hm[h][e] = table[e][h]: the bias table head-major, so that a unit's slice is
// contiguous for the backward kernels, which read it as `table`
__global__ __launch_bounds__(256) void bias_heads_kernel(int ts, int heads, const float* __restrict__ table,
                                                         float* __restrict__ hm) {
    const int idx = blockIdx.x * 256 + threadIdx.x; // h * ts + e
    if (idx >= ts * heads) return;
    const int h = idx / ts, e = idx - h * ts;
    hm[idx] = table[(size_t)e * heads + h];
}

// ---- host side
// bytes of the head-major table copy at the front of the workspace or scratch
static size_t bias_heads_bytes(const Geometry& g) {
    return ((size_t)g.heads * g.table_size * sizeof(float) + 255) / 256 * 256;
}
static hipError_t launch_bias_heads(const Geometry& g, const float* table, float* hm, hipStream_t s) {
    const int n = g.heads * g.table_size;
    hipLaunchKernelGGL(bias_heads_kernel, dim3((n + 255) / 256), dim3(256), 0, s, g.table_size, g.heads, table, hm);
    return hipGetLastError();
}

// the single-workgroup bf16 kernel, or else the two big-window kernels
static bool bwd_small_fits(const Geometry& g) {
    return (g.N + 15) / 16 <= kBwdMaxTiles && bwd_lds(g).total <= (size_t)kLdsBytes;
}

static bool bwd_big_fits(const Geometry& g) {
    const BwdBigLds L = bwd_big_lds(g, bwd_kv_waves(g.head_dim));
    return L.total_q <= (size_t)kLdsBytes && L.total_k <= (size_t)kLdsBytes;
}

#ifndef SWA_BWD_KVP
#define SWA_BWD_KVP 1
#endif

// The persistent key kernel (pair sums over windows): big windows of 5 to 9
// query blocks (129 to 288 tokens) with heads of 32 or 64.
static bool bwd_kvp_fits(const Geometry& g) {
    if (!SWA_BWD_KVP || bwd_small_fits(g) || !bwd_big_fits(g)) return false;
    if (g.head_dim != 32 && g.head_dim != 64) return false;
    const int NB = kvp_lds(g).NPX / kBwdBlk;
    return NB >= 5 && NB <= kKvpBlocks && kvp_lds(g).total <= (size_t)kLdsBytes;
}

// Key groups of a window, and runs of windows per (head, group): enough
// workgroups for one per compute unit, never more runs than windows.
struct KvpPlan {
    int groups, runs;
};
static KvpPlan kvp_plan(const Geometry& g, int64_t windows) {
    KvpPlan p;
    p.groups = (kvp_lds(g).NPX / 16 + kKvpTiles - 1) / kKvpTiles;
    const int64_t r = kKvpWorkgroups / ((int64_t)g.heads * p.groups);
    p.runs = (int)(r < 1 ? 1 : r > windows ? (windows < 1 ? 1 : windows) : r);
    return p;
}
// floats of the kernel's workgroup sums and of their sums over runs
static size_t kvp_sums_floats(const Geometry& g, const KvpPlan& p) {
    return (size_t)g.heads * p.groups * p.runs * kKvpSums;
}
static size_t kvp_pairs_floats(const Geometry& g, const KvpPlan& p) {
    return p.runs > 1 ? (size_t)g.heads * p.groups * kKvpSums : 0;
}

bool backward_fits(const Geometry& g, bool bf16) {
    if (!bf16) return g.head_dim <= 64 && f32_bwd_lds_bytes(g) <= (size_t)kLdsBytes;
    const int64_t rows = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    return rows < kRowMask && (bwd_small_fits(g) || bwd_big_fits(g));
}

int backward_schedule(const Geometry& g, bool bf16) {
    if (!backward_fits(g, bf16)) return 0;
    return !bf16 || bwd_small_fits(g) ? 1 : 2;
}

static size_t backward_work_bytes(const Geometry& g);
size_t backward_workspace_bytes(const Geometry& g) {
    return bias_heads_bytes(g) + backward_work_bytes(g);
}

// the workspace after the head-major table
static size_t backward_work_bytes(const Geometry& g) {
    if (bwd_kvp_fits(g)) { // per-query statistics, workgroup sums, their sums over runs
        const KvpPlan p = kvp_plan(g, g.windows);
        return ((size_t)(g.windows * g.heads) * 2 * kvp_lds(g).NPX + kvp_sums_floats(g, p) +
                kvp_pairs_floats(g, p)) * sizeof(float);
    }
    const size_t units = (size_t)(g.windows * g.heads) * g.table_size;
    const size_t chunks = (size_t)kDtableChunks * g.heads * g.table_size;
    // big windows: per query, lse2 and D
    const size_t stats =
        bwd_small_fits(g) ? 0 : (size_t)(g.windows * g.heads) * 2 * bwd_big_lds(g, bwd_kv_waves(g.head_dim)).NPX;
    return (units + chunks + stats) * sizeof(float);
}

typedef void (*bwd_bf16_t)(Geometry, const uint16_t*, const uint16_t*, const uint16_t*, const float*,
                           const uint16_t*, uint16_t*, uint16_t*, uint16_t*, float*, uint32_t, uint32_t);

static bwd_bf16_t bwd_bf16_variant(const Geometry& g) {
    const bool bv = g.win[2] % 4 == 0;
    if (g.head_dim == 32) return bv ? attn_bf16_bwd_kernel<32, true> : attn_bf16_bwd_kernel<32, false>;
    if (g.head_dim == 128) return bv ? attn_bf16_bwd_kernel<128, true> : attn_bf16_bwd_kernel<128, false>;
    return bv ? attn_bf16_bwd_kernel<64, true> : attn_bf16_bwd_kernel<64, false>;
}

static bwd_bf16_t bwd_bf16_pvariant(const Geometry& g) {
    const bool bv = g.win[2] % 4 == 0;
    if (g.head_dim == 32) return bv ? attn_bf16_bwd_pkernel<32, true> : attn_bf16_bwd_pkernel<32, false>;
    if (g.head_dim == 128) return bv ? attn_bf16_bwd_pkernel<128, true> : attn_bf16_bwd_pkernel<128, false>;
    return bv ? attn_bf16_bwd_pkernel<64, true> : attn_bf16_bwd_pkernel<64, false>;
}

#ifndef SWA_BWD_PERSISTENT
#define SWA_BWD_PERSISTENT 1
#endif

hipError_t backward_plan(const Geometry& g, bool bf16, int* blocks) {
    *blocks = 0;
    if (bf16 && bwd_kvp_fits(g)) { // the persistent key kernel's workgroups
        const KvpPlan p = kvp_plan(g, g.windows);
        *blocks = g.heads * p.groups * p.runs;
        return hipSuccess;
    }
    if (!SWA_BWD_PERSISTENT || !bf16 || !bwd_small_fits(g) || bwd_plds(g).total > (size_t)kLdsBytes)
        return hipSuccess;
    int per_cu = 0, dev = 0, cus = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)bwd_bf16_pvariant(g),
                                                                (kBwdWaves + kBwdPLoaders) * 64, bwd_plds(g).total);
    if (e != hipSuccess) return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int n = per_cu * cus / kXcds * kXcds;
    *blocks = n > 0 ? n : 0;
    return hipSuccess;
}

// Compute waves of the query kernel (16 queries each).  Heads of up to 64:
// whichever of 4, 6 and 8 waves leaves the fewest idle query slots in the
// last block, ties to more waves (fewer re-reads of K and V).  128-wide heads:
// 6 for windows of 512 tokens or more, so that two workgroups of 8 waves fit a
// CU's registers, 4 below.
static int bwd_q_waves(const Geometry& g) {
    if (g.head_dim == 128) return g.N < 512 ? 4 : 6;
    int best = 4, idle = 1 << 30;
    for (int qw : {4, 6, 8}) {
        const int slots = (g.N + qw * 16 - 1) / (qw * 16) * (qw * 16);
        if (slots - g.N <= idle) {
            idle = slots - g.N;
            best = qw;
        }
    }
    return best;
}

hipError_t prepare_backward_kernels(int max_lds) {
    const void* fs[] = {(const void*)attn_bf16_bwd_pkernel<32, true>, (const void*)attn_bf16_bwd_pkernel<32, false>,
                        (const void*)attn_bf16_bwd_pkernel<64, true>, (const void*)attn_bf16_bwd_pkernel<64, false>,
                        (const void*)attn_bf16_bwd_pkernel<128, true>, (const void*)attn_bf16_bwd_pkernel<128, false>,
                        (const void*)attn_bf16_bwd_kernel<32, true>,  (const void*)attn_bf16_bwd_kernel<32, false>,
                        (const void*)attn_bf16_bwd_kernel<64, true>,  (const void*)attn_bf16_bwd_kernel<64, false>,
                        (const void*)attn_bf16_bwd_kernel<128, true>, (const void*)attn_bf16_bwd_kernel<128, false>,
                        (const void*)attn_f32_bwd_kernel<32>,         (const void*)attn_f32_bwd_kernel<64>,
                        (const void*)attn_bf16_bwd_q_kernel<32, 4>,   (const void*)attn_bf16_bwd_q_kernel<64, 4>,
                        (const void*)attn_bf16_bwd_q_kernel<128, 4>,  (const void*)attn_bf16_bwd_q_kernel<32, 8>,
                        (const void*)attn_bf16_bwd_q_kernel<64, 8>,   (const void*)attn_bf16_bwd_q_kernel<128, 6>,
                        (const void*)attn_bf16_bwd_q_kernel<32, 6>,   (const void*)attn_bf16_bwd_q_kernel<64, 6>,
                        (const void*)attn_bf16_bwd_kv_kernel<32, 6, 0>,  (const void*)attn_bf16_bwd_kv_kernel<32, 6, 1>,
                        (const void*)attn_bf16_bwd_kv_kernel<32, 6, 2>,  (const void*)attn_bf16_bwd_kv_kernel<64, 6, 0>,
                        (const void*)attn_bf16_bwd_kv_kernel<64, 6, 1>,  (const void*)attn_bf16_bwd_kv_kernel<64, 6, 2>,
                        (const void*)attn_bf16_bwd_kv_kernel<128, 8, 0>, (const void*)attn_bf16_bwd_kv_kernel<128, 8, 1>,
                        (const void*)attn_bf16_bwd_kv_kernel<128, 8, 2>, (const void*)attn_bf16_bwd_kvp_kernel<32, 2>,
                        (const void*)attn_bf16_bwd_kvp_kernel<32, 3>, (const void*)attn_bf16_bwd_kvp_kernel<64, 2>,
                        (const void*)attn_bf16_bwd_kvp_kernel<64, 3>};
    for (const void* f : fs) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The key kernel for g: the head width, and how a tile diagonal of the table
// gradient splits into runs (window widths that are multiples of 16 never
// split it; widths of at least 8 split it at row starts only).
typedef void (*kv_t)(Geometry, const uint16_t*, const uint16_t*, const uint16_t*, const float*, const uint16_t*,
                     uint16_t*, uint16_t*, const float*, float*, uint32_t, uint32_t);

template <int D, int KW>
static kv_t bwd_kv_runs(const Geometry& g) {
    if (g.win[2] % 16 == 0) return attn_bf16_bwd_kv_kernel<D, KW, 0>;
    if (g.win[2] >= 8) return attn_bf16_bwd_kv_kernel<D, KW, 1>;
    return attn_bf16_bwd_kv_kernel<D, KW, 2>;
}

static kv_t bwd_kv_variant(const Geometry& g) {
    if (g.head_dim == 32) return bwd_kv_runs<32, 6>(g);
    if (g.head_dim == 64) return bwd_kv_runs<64, 6>(g);
    return bwd_kv_runs<128, 8>(g);
}

// The attention gradients of units work0 .. work0 + count - 1: dq, dk, dv of
// their tokens, their table-gradient shares at units[(unit - work0) * ts] and,
// for big windows, their per-query statistics at stats[(unit - work0) * 2 NPX].
// The big-window query kernel over units work0 .. work0 + count - 1: dq, and
// each unit's per-query statistics at stats[(unit - work0) * 2 NPX].
static hipError_t launch_big_query(const Geometry& g, const void* q, const void* k, const void* v, const float* table,
                                   const void* dout, void* dq, uint32_t work0, uint32_t count, float* stats,
                                   const void* o, const float* lse, hipStream_t s) {
    const BwdBigLds L = bwd_big_lds(g, bwd_kv_waves(g.head_dim));
    const int QW = bwd_q_waves(g);
    const dim3 qgrid(count * (unsigned)((g.N + QW * 16 - 1) / (QW * 16)));
    typedef void (*qk_t)(Geometry, const uint16_t*, const uint16_t*, const uint16_t*, const float*,
                         const uint16_t*, uint16_t*, float*, uint32_t, uint32_t, const uint16_t*, const float*);
    const qk_t fq = g.head_dim == 128 ? (QW == 6 ? attn_bf16_bwd_q_kernel<128, 6> : attn_bf16_bwd_q_kernel<128, 4>)
                    : g.head_dim == 64
                        ? (QW == 8   ? attn_bf16_bwd_q_kernel<64, 8>
                           : QW == 6 ? attn_bf16_bwd_q_kernel<64, 6>
                                     : attn_bf16_bwd_q_kernel<64, 4>)
                        : (QW == 8   ? attn_bf16_bwd_q_kernel<32, 8>
                           : QW == 6 ? attn_bf16_bwd_q_kernel<32, 6>
                                     : attn_bf16_bwd_q_kernel<32, 4>);
    hipLaunchKernelGGL(fq, qgrid, dim3((QW + kBwdLoaders) * 64), L.total_q, s, g, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, table, (const uint16_t*)dout, (uint16_t*)dq, stats,
                       work0, count, (const uint16_t*)o, lse);
    return hipGetLastError();
}

// The persistent key kernel over windows w0 .. w0 + nw - 1 (statistics of
// their units at stats, as launch_big_query leaves them), then the table
// gradient from its pair sums: dtable = (accumulate ? dtable : 0) + the
// windows' share.  sums: kvp_sums_floats, pairs: kvp_pairs_floats (runs > 1).
static hipError_t launch_kvp(const Geometry& g, const void* q, const void* k, const void* v, const float* table,
                             const void* dout, void* dk, void* dv, float* dtable, const float* stats, float* sums,
                             float* pairs, uint32_t w0, uint32_t nw, const KvpPlan& p, int accumulate,
                             hipStream_t s) {
    const unsigned wgs = (unsigned)(g.heads * p.runs * p.groups);
    const bool sb3 = kvp_step_blocks(kvp_lds(g).NPX / kBwdBlk) == 3;
    hipLaunchKernelGGL(g.head_dim == 32 ? (sb3 ? attn_bf16_bwd_kvp_kernel<32, 3> : attn_bf16_bwd_kvp_kernel<32, 2>)
                                        : (sb3 ? attn_bf16_bwd_kvp_kernel<64, 3> : attn_bf16_bwd_kvp_kernel<64, 2>),
                       dim3(wgs),
                       dim3((kKvpWaves + kKvpLoaders) * 64), kvp_lds(g).total, s, g, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, table, (const uint16_t*)dout, (uint16_t*)dk,
                       (uint16_t*)dv, stats, sums, w0, nw, p.runs, p.groups);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float* ps = sums;
    if (p.runs > 1) {
        const int64_t n = (int64_t)g.heads * p.groups * kKvpSums;
        hipLaunchKernelGGL(pair_runs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g.heads, p.runs,
                           p.groups, (const float*)sums, pairs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        ps = pairs;
    }
    const int n = g.heads * g.table_size; // a wave per entry, four per block
    hipLaunchKernelGGL(dtable_pairs_kernel, dim3((n + 3) / 4), dim3(256), 0, s, g, p.groups, ps, dtable,
                       accumulate);
    return hipGetLastError();
}

static hipError_t launch_backward_units(const Geometry& g, bool bf16, const void* q, const void* k, const void* v,
                                        const float* table, const void* dout, void* dq, void* dk, void* dv,
                                        uint32_t work0, uint32_t count, float* units, float* stats, const void* o,
                                        const float* lse, int blocks, hipStream_t s) {
    const dim3 grid(count);
    if (bf16 && !bwd_small_fits(g)) {
        const BwdBigLds L = bwd_big_lds(g, bwd_kv_waves(g.head_dim));
        const int KW = bwd_kv_waves(g.head_dim);
        const kv_t fk = bwd_kv_variant(g);
        hipError_t e = launch_big_query(g, q, k, v, table, dout, dq, work0, count, stats, o, lse, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fk, grid, dim3((KW + kBwdLoaders) * 64), L.total_k, s, g, (const uint16_t*)q, (const uint16_t*)k,
                           (const uint16_t*)v, table, (const uint16_t*)dout, (uint16_t*)dk, (uint16_t*)dv,
                           (const float*)stats, units, work0, count);
    } else if (bf16 && blocks > 0) {
        hipLaunchKernelGGL(bwd_bf16_pvariant(g), dim3((unsigned)blocks), dim3((kBwdWaves + kBwdPLoaders) * 64),
                           bwd_plds(g).total, s, g, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, table,
                           (const uint16_t*)dout, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, units, work0, count);
    } else if (bf16) {
        hipLaunchKernelGGL(bwd_bf16_variant(g), grid, dim3(kBwdWaves * 64), bwd_lds(g).total, s, g,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, table, (const uint16_t*)dout,
                           (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, units, work0, count);
    } else if (g.head_dim == 32) {
        hipLaunchKernelGGL(attn_f32_bwd_kernel<32>, grid, dim3(kF32BwdThreads), f32_bwd_lds_bytes(g), s, g,
                           (const float*)q, (const float*)k, (const float*)v, table, (const float*)dout, (float*)dq,
                           (float*)dk, (float*)dv, units, work0, count);
    } else {
        hipLaunchKernelGGL(attn_f32_bwd_kernel<64>, grid, dim3(kF32BwdThreads), f32_bwd_lds_bytes(g), s, g,
                           (const float*)q, (const float*)k, (const float*)v, table, (const float*)dout, (float*)dq,
                           (float*)dk, (float*)dv, units, work0, count);
    }
    return hipGetLastError();
}

hipError_t launch_backward(const Geometry& g, bool bf16, const void* q, const void* k, const void* v,
                           const float* table_in, const void* dout, void* dq, void* dk, void* dv, float* dtable,
                           void* workspace_in, const void* o, const float* lse, int blocks, hipStream_t s) {
    float* table = (float*)workspace_in; // the head-major copy that every kernel below reads
    void* workspace = (unsigned char*)workspace_in + bias_heads_bytes(g);
    {
        const hipError_t e = launch_bias_heads(g, table_in, table, s);
        if (e != hipSuccess) return e;
    }
    if (bf16 && bwd_kvp_fits(g)) {
        const KvpPlan p = kvp_plan(g, g.windows);
        float* stats = (float*)workspace;
        float* sums = stats + (size_t)(g.windows * g.heads) * 2 * kvp_lds(g).NPX;
        float* pairs = sums + kvp_sums_floats(g, p);
        hipError_t e = launch_big_query(g, q, k, v, table, dout, dq, 0, (uint32_t)(g.windows * g.heads), stats, o,
                                        lse, s);
        if (e != hipSuccess) return e;
        return launch_kvp(g, q, k, v, table, dout, dk, dv, dtable, stats, sums, pairs, 0, (uint32_t)g.windows, p, 0,
                          s);
    }
    float* units = (float*)workspace;
    float* chunks = units + (size_t)(g.windows * g.heads) * g.table_size;
    float* stats = chunks + (size_t)kDtableChunks * g.heads * g.table_size;
    hipError_t e = launch_backward_units(g, bf16, q, k, v, table, dout, dq, dk, dv, 0,
                                         (uint32_t)(g.windows * g.heads), units, stats, o, lse, blocks, s);
    if (e != hipSuccess) return e;
    const int n = g.heads * g.table_size;
    hipLaunchKernelGGL(dtable_chunk_kernel, dim3((n + 255) / 256, kDtableChunks), dim3(256), 0, s, g.windows,
                       g.heads, g.table_size, (const float*)units, chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(dtable_sum_kernel, dim3((n + 255) / 256), dim3(256), 0, s, g.heads, g.table_size,
                       (const float*)chunks, dtable);
    return hipGetLastError();
}

// ---- the backward pass through a fixed scratch buffer, in passes over runs
// of whole window chunks (the chunks of dtable_chunk_kernel).  After each pass
// the chunks it covered are summed and added to the running table gradient,
// chunk by chunk in order, which is exactly the sum dtable_sum_kernel forms:
// the results equal the workspace path's bit for bit.

// Bytes of scratch one window needs: its heads' table shares (and per-query
// statistics of big windows).
static size_t scratch_per_window(const Geometry& g, bool bf16) {
    size_t per_unit = (size_t)g.table_size;
    if (bf16 && !bwd_small_fits(g)) per_unit += 2 * (size_t)bwd_big_lds(g, bwd_kv_waves(g.head_dim)).NPX;
    return per_unit * g.heads * sizeof(float);
}

static int64_t chunk_window(const Geometry& g, int c) { return g.windows * c / kDtableChunks; }

// The persistent key kernel through the scratch: passes over runs of windows,
// each with the statistics of its units, the workgroup sums and their sums.
// The runs per (head, group) are halved until a pass holds at least two
// windows per run; the smallest layout is one run of one window.
static size_t kvp_window_bytes(const Geometry& g) { return (size_t)g.heads * 2 * kvp_lds(g).NPX * sizeof(float); }
static size_t kvp_fixed_bytes(const Geometry& g, const KvpPlan& p) {
    return (kvp_sums_floats(g, p) + kvp_pairs_floats(g, p)) * sizeof(float);
}

static size_t scratch_work_bytes(const Geometry& g, bool bf16);
size_t backward_scratch_bytes(const Geometry& g, bool bf16) { return bias_heads_bytes(g) + scratch_work_bytes(g, bf16); }

static size_t scratch_work_bytes(const Geometry& g, bool bf16) {
    if (bf16 && bwd_kvp_fits(g)) {
        KvpPlan p = kvp_plan(g, 1);
        p.runs = 1;
        return kvp_window_bytes(g) + kvp_fixed_bytes(g, p);
    }
    int64_t most = 0; // windows of the largest chunk
    for (int c = 0; c < kDtableChunks; c++) {
        const int64_t n = chunk_window(g, c + 1) - chunk_window(g, c);
        most = n > most ? n : most;
    }
    return (size_t)most * scratch_per_window(g, bf16);
}

// dtable[e][h] = (c0 == 0 ? 0 : dtable[e][h]) + chunk sums c0 .. c1 - 1 in order;
// the shares of windows w0 .. are at units[(w - w0) * heads * ts].
__global__ __launch_bounds__(256) void dtable_accumulate_kernel(int64_t windows, int heads, int ts, int c0, int c1,
                                                                int64_t w0, const float* __restrict__ units,
                                                                float* __restrict__ dtable) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x; // h * ts + e
    if (idx >= heads * ts) return;
    const int h = idx / ts, e = idx - h * ts;
    float run = c0 == 0 ? 0.f : dtable[(size_t)e * heads + h];
    for (int c = c0; c < c1; c++) {
        const int64_t a = windows * c / kDtableChunks, b = windows * (c + 1) / kDtableChunks;
        float acc = 0.f;
        for (int64_t w = a; w < b; w++) acc += units[(size_t)(w - w0) * heads * ts + idx];
        run += acc;
    }
    dtable[(size_t)e * heads + h] = run;
}

hipError_t launch_backward_scratch(const Geometry& g, bool bf16, const void* q, const void* k, const void* v,
                                   const float* table_in, const void* dout, void* dq, void* dk, void* dv,
                                   float* dtable, void* scratch_in, size_t scratch_in_bytes, int blocks,
                                   hipStream_t s) {
    if (scratch_in_bytes < bias_heads_bytes(g)) return hipErrorInvalidValue; // checked by the caller
    float* table = (float*)scratch_in; // the head-major copy that every kernel below reads
    void* scratch = (unsigned char*)scratch_in + bias_heads_bytes(g);
    const size_t scratch_bytes = scratch_in_bytes - bias_heads_bytes(g);
    {
        const hipError_t e = launch_bias_heads(g, table_in, table, s);
        if (e != hipSuccess) return e;
    }
    if (bf16 && bwd_kvp_fits(g)) {
        KvpPlan p = kvp_plan(g, g.windows);
        int64_t per_pass = 0;
        for (;;) {
            const size_t fixed = kvp_fixed_bytes(g, p);
            per_pass = fixed < scratch_bytes ? (int64_t)((scratch_bytes - fixed) / kvp_window_bytes(g)) : 0;
            if (per_pass >= g.windows || per_pass >= 2 * (int64_t)p.runs || p.runs == 1) break;
            p.runs = p.runs / 2;
        }
        if (per_pass < 1) return hipErrorInvalidValue; // the caller checks backward_scratch_bytes first
        per_pass = per_pass < g.windows ? per_pass : g.windows;
        for (int64_t w0 = 0; w0 < g.windows; w0 += per_pass) {
            const int64_t nw = g.windows - w0 < per_pass ? g.windows - w0 : per_pass;
            KvpPlan pp = p;
            pp.runs = (int)(pp.runs < nw ? pp.runs : nw);
            float* stats = (float*)scratch;
            float* sums = stats + (size_t)nw * g.heads * 2 * kvp_lds(g).NPX;
            float* pairs = sums + kvp_sums_floats(g, pp);
            hipError_t e = launch_big_query(g, q, k, v, table, dout, dq, (uint32_t)(w0 * g.heads),
                                            (uint32_t)(nw * g.heads), stats, nullptr, nullptr, s);
            if (e != hipSuccess) return e;
            e = launch_kvp(g, q, k, v, table, dout, dk, dv, dtable, stats, sums, pairs, (uint32_t)w0, (uint32_t)nw,
                           pp, w0 > 0, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const size_t per_window = scratch_per_window(g, bf16);
    const int n = g.heads * g.table_size;
    int c0 = 0;
    while (c0 < kDtableChunks) {
        // the longest run of chunks whose windows' shares fit the scratch
        int c1 = c0 + 1;
        while (c1 < kDtableChunks &&
               (size_t)(chunk_window(g, c1 + 1) - chunk_window(g, c0)) * per_window <= scratch_bytes)
            c1++;
        const int64_t w0 = chunk_window(g, c0), w1 = chunk_window(g, c1);
        float* units = (float*)scratch;
        float* stats = units + (size_t)(w1 - w0) * g.heads * g.table_size;
        hipError_t e;
        if (w1 > w0) {
            e = launch_backward_units(g, bf16, q, k, v, table, dout, dq, dk, dv, (uint32_t)(w0 * g.heads),
                                      (uint32_t)((w1 - w0) * g.heads), units, stats, nullptr, nullptr, blocks, s);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(dtable_accumulate_kernel, dim3((n + 255) / 256), dim3(256), 0, s, g.windows, g.heads,
                           g.table_size, c0, c1, w0, (const float*)units, dtable);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        c0 = c1;
    }
    return hipSuccess;
}

} // namespace swa
