// Window geometry shared by the library's kernels and host code.
//
// A token of the padded (time, latitude, longitude) grid is addressed by the
// window it falls in after the grid is rolled by -shift, and by its row-major
// position n inside that window (TERRA page: abstract, window layouts and
// shifted-window execution; Table I, padded resolution).  For window
// coordinates W_a and local coordinates l_a:
//   rolled coordinate  c'_a = W_a * w_a + l_a
//   source coordinate  c_a  = (c'_a + s_a) mod P_a      (pad when c_a >= E_a)
//   wrapped            c'_a >= P_a - s_a, on masked axes only
// Two tokens of one window may attend each other when neither is pad and
// their wrapped flags agree on every masked axis.  The relative-position bias
// of (query n, key m) sits at table index qb(n) - kb(m) with
//   qb = (l_t + w_t - 1) * Dy * Dx + (l_y + w_y - 1) * Dx + (l_x + w_x - 1)
//   kb =  l_t * Dy * Dx + l_y * Dx + l_x,         Dy = 2 w_y - 1, Dx = 2 w_x - 1
// so that qb - kb = (l_t(n) - l_t(m) + w_t - 1) * Dy * Dx + ... (query minus key).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

// n / d for 0 <= n < 2^31 and 1 <= d < 2^31 by multiply-high and shift
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): t = mulhi(m, n), q = (t + n) >> l.
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) l++;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

__host__ __device__ inline uint32_t fdiv(const FastDiv& f, uint32_t n) {
    const uint32_t t = (uint32_t)(((uint64_t)f.m * n) >> 32);
    return (t + n) >> f.l;
}

struct Geometry {
    int batch, heads, head_dim;
    int ext[3];   // real extents (T, H, W)
    int pad[3];   // padded extents
    int win[3];   // window
    int shift[3]; // shift
    int cyc[3];   // 1 = cyclic axis
    int nwin[3];  // pad / win
    int N;        // tokens per window
    int nW;       // windows per batch item
    int64_t windows; // batch * nW
    int row;      // elements per token: heads * head_dim
    int tdy, tdx; // 2 w_y - 1, 2 w_x - 1
    int table_size; // (2 w_t - 1) * tdy * tdx
    int c0;       // qb - kb of any token (see above)
    float scale;  // logit scale
    FastDiv fd_heads, fd_nW, fd_nwin1, fd_nwin2, fd_win1, fd_win2;
};

// Whether any key of window (wc) can be hidden from some query: the window
// holds the wrapped part of a masked axis, or pad tokens.  A rolled window
// [lo, lo + w) takes sources [lo + s, min(lo + w + s, P)) and, past the wrap,
// [0, lo + w + s - P); pad is any source >= E.
__host__ __device__ inline bool window_maybe_masked(const Geometry& g, const int wc[3]) {
    for (int a = 0; a < 3; a++) {
        if (g.cyc[a]) continue;
        const int lo = wc[a] * g.win[a];
        const int hi = lo + g.win[a] + g.shift[a];
        if (g.shift[a] > 0 && wc[a] == g.nwin[a] - 1) return true;
        if ((hi < g.pad[a] ? hi : g.pad[a]) > g.ext[a]) return true;
        if (hi - g.pad[a] > g.ext[a]) return true;
    }
    return false;
}

// Mask words.  A key word holds kb in bits 0..15, the wrapped flags of the
// masked axes in bits 16..18 and the pad flag in bit 19.  A query word holds
// qb in bits 0..15 and, in bits 16..24, its wrapped flags (or 0x100 for a pad
// query, which then matches no key).  Key m is visible to query n exactly
// when (key_word >> 16) == (query_word >> 16).
constexpr int kPadBit = 1 << 19;
constexpr int kNoKey = 0xF << 16;      // key word of a slot past N
constexpr int kPadQuery = 0x100 << 16; // region field of a pad query

struct TokenInfo {
    int64_t tok; // flat real token index ((b*T + t)*H + y)*W + x, or -1 for pad
    int region;  // wrapped flags of the masked axes (bit a for axis a)
    int kb, qb;  // bias offsets (see above)
};

__host__ __device__ inline void window_coords(const Geometry& g, int64_t wi, int& b, int wc[3]) {
    b = (int)(wi / g.nW);
    int r = (int)(wi - (int64_t)b * g.nW);
    wc[2] = r % g.nwin[2];
    r /= g.nwin[2];
    wc[1] = r % g.nwin[1];
    wc[0] = r / g.nwin[1];
}

__host__ __device__ inline TokenInfo token_info(const Geometry& g, int b, const int wc[3], int n) {
    int l[3];
    l[2] = n % g.win[2];
    int r = n / g.win[2];
    l[1] = r % g.win[1];
    l[0] = r / g.win[1];
    TokenInfo ti;
    int64_t tok = b;
    bool is_pad = false;
    ti.region = 0;
    for (int a = 0; a < 3; a++) {
        int cr = wc[a] * g.win[a] + l[a];
        int c = cr + g.shift[a];
        if (c >= g.pad[a]) c -= g.pad[a];
        if (c >= g.ext[a]) is_pad = true;
        if (!g.cyc[a] && cr >= g.pad[a] - g.shift[a]) ti.region |= 1 << a;
        tok = tok * g.ext[a] + c;
    }
    ti.tok = is_pad ? -1 : tok;
    ti.kb = (l[0] * g.tdy + l[1]) * g.tdx + l[2];
    ti.qb = ((l[0] + g.win[0] - 1) * g.tdy + (l[1] + g.win[1] - 1)) * g.tdx + (l[2] + g.win[2] - 1);
    return ti;
}

__host__ __device__ inline int key_word(const TokenInfo& ti) {
    return ti.kb | (ti.region << 16) | (ti.tok < 0 ? kPadBit : 0);
}

__host__ __device__ inline int query_word(const TokenInfo& ti) {
    return ti.qb | (ti.tok < 0 ? kPadQuery : (ti.region << 16));
}

__host__ __device__ inline bool visible(int qword, int kword) {
    return (qword >> 16) == (kword >> 16);
}

// Launchers (swa_kernels.hip).  All return the launch status.
hipError_t launch_gather(const Geometry& g, int elem_bytes, const void* src, void* dst,
                         hipStream_t s);
hipError_t launch_scatter(const Geometry& g, int elem_bytes, const void* src, void* dst,
                          hipStream_t s);
hipError_t launch_visibility(const Geometry& g, int64_t window, uint8_t* out, hipStream_t s);
// With lse (fused layout only; may be null) every real query's log-sum-exp of
// its logits also goes to lse[row * heads + head].
hipError_t launch_attention_f32(const Geometry& g, bool staged, const float* q, const float* k,
                                const float* v, const float* table, float* out, float* lse, hipStream_t s);
// The per-unit schedule (stream false) first refreshes bias_hm, a head-major
// copy of table (bf16_kblock_workspace_bytes), and reads its slices from it.
hipError_t launch_attention_bf16(const Geometry& g, bool stream, int blocks, bool staged, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const float* table, float* bias_hm,
                                 uint16_t* out, float* lse, hipStream_t s);
// LDS bytes the attention kernels need for g (bf16: the smallest among the
// schedules that take the window; (size_t)-1 when none does).
size_t attention_lds_bytes(const Geometry& g, bool bf16, bool staged);
// Whether the streaming bf16 schedule (persistent blocks, two LDS stages) fits,
// for the fused or the staged variant.
bool bf16_stream_fits(const Geometry& g, bool staged);
// Whether the per-unit bf16 schedule (a window's K and V in one workgroup's LDS) fits.
bool bf16_block_fits(const Geometry& g);
// Workgroups one bf16 attention launch uses (0: the kernel does not fit).
hipError_t bf16_plan(const Geometry& g, bool stream, int* blocks);
// Key-blocked bf16 schedule (windows of any size): whether its LDS ring fits,
// the head-major bias copy it needs (bytes), its workgroup count (0: does not
// fit) and its launch (which first refreshes the bias copy from table).
bool bf16_kblock_fits(const Geometry& g);
size_t bf16_kblock_workspace_bytes(const Geometry& g);
hipError_t kblock_plan(const Geometry& g, int* blocks);
hipError_t launch_attention_kblock(const Geometry& g, bool staged, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const float* table, float* bias_hm, uint16_t* out,
                                   float* lse, hipStream_t s);
// Lets every attention kernel take up to max_lds bytes of dynamic LDS.
hipError_t prepare_kernels(int max_lds);

} // namespace swa
