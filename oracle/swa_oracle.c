/*
 * Plain fp64 CPU reference ("oracle") for the forward pass of shifted-window
 * multi-head self-attention over a (time, latitude, longitude) token grid.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library and includes nothing from it.
 *
 * What it computes (the "direct form").  Sources: the TERRA page
 * ("TERRA: A Hierarchical Parallel Training and Memory Orchestration Framework
 * for High-Resolution AI-based Earth Modeling"): the abstract (window-based
 * Swin attention replaces global attention; shifted-window execution; tokens
 * are routed into window layouts for the Transformer and back), Table I
 * (real resolution H, W and padded resolution H^, W^; embedding d), Table V
 * (heads N_h, window size w) and the Fig. 5 caption (shift token routes).
 * The pages print no formula; every reading taken where they are silent is
 * listed with the repository's design notes, and restated at each step here.
 *
 * For every batch b, head h and REAL query token i = (t, y, x):
 *   - On each axis a (extent E, padded extent P >= E, window w, shift s):
 *       * cyclic axis (longitude; P == E): the key segment of coordinate c is
 *         every c2 with floor(((c2 - s) mod E) / w) == floor(((c - s) mod E) / w);
 *       * masked axis (time, latitude): the key segment of c is the block of
 *         [0, P) cut at 0 and at s + k*w (k >= 0) that holds c, intersected
 *         with the real range [0, E) (pad, placed at the end of the axis, is
 *         never a key).
 *     The key set K(i) is the product of the three per-axis segments.  This
 *     is what rolling the padded grid by -s, cutting it into w-sized windows
 *     and masking pairs that straddle the wrap of a masked axis gives.
 *   - Window-local coordinate: l_a(c) = ((c - s) mod P) mod w.
 *   - logit(i, j) = scale * <q_i, k_j>
 *                   + table[l_t(i)-l_t(j)+w_t-1][l_y(i)-l_y(j)+w_y-1]
 *                          [l_x(i)-l_x(j)+w_x-1][h]      for j in K(i)
 *   - o_i = sum_{j in K(i)} softmax_j(logit(i, .)) v_j, with max subtraction.
 * i is in K(i), so no denominator is zero.
 *
 * Inputs are float (fp32 holds every bf16 value exactly); all arithmetic is
 * double.  Layouts: q, k, v are [B][T][H][W][heads][head_dim] over the REAL
 * extents, C-contiguous; table is [2w_t-1][2w_y-1][2w_x-1][heads].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int batch, heads, head_dim;
    int extent[3]; /* real T, H, W */
    int padded[3]; /* padded T^, H^, W^ */
    int window[3];
    int shift[3];
    int cyclic[3]; /* 1: cyclic axis, 0: masked axis */
    double scale;
} swo_problem;

static long pos_mod(long a, long m) {
    long r = a % m;
    return r < 0 ? r + m : r;
}

/* Which key segment coordinate c falls in, on axis a (see header). */
static long segment_label(const swo_problem* p, int a, long c) {
    long w = p->window[a], s = p->shift[a];
    if (p->cyclic[a]) return pos_mod(c - s, p->extent[a]) / w;
    if (c < s) return -1; /* the head block [0, s) */
    return (c - s) / w;
}

/* Position of coordinate c inside its rolled window, on axis a. */
long swo_local_coord(const swo_problem* p, int a, long c) {
    return pos_mod(c - p->shift[a], p->padded[a]) % p->window[a];
}

/* 1 iff the key at padded-frame coordinates kc is visible to the query at qc:
 * both real, and in the same segment on every axis. */
int swo_visible(const swo_problem* p, const long* qc, const long* kc) {
    for (int a = 0; a < 3; a++) {
        if (qc[a] < 0 || qc[a] >= p->padded[a] || kc[a] < 0 || kc[a] >= p->padded[a]) return 0;
        if (qc[a] >= p->extent[a] || kc[a] >= p->extent[a]) return 0;
        if (segment_label(p, a, qc[a]) != segment_label(p, a, kc[a])) return 0;
    }
    return 1;
}

/* Checks the problem describes a well-formed tiling; 0 on success. */
int swo_check(const swo_problem* p) {
    if (p->batch < 1 || p->heads < 1 || p->head_dim < 1) return 1;
    for (int a = 0; a < 3; a++) {
        if (p->extent[a] < 1 || p->padded[a] < p->extent[a]) return 2;
        if (p->window[a] < 1 || p->window[a] > p->padded[a]) return 3;
        if (p->padded[a] % p->window[a] != 0) return 4;
        if (p->shift[a] < 0 || p->shift[a] >= p->window[a]) return 5;
        if (p->cyclic[a] && p->padded[a] != p->extent[a]) return 6;
    }
    return 0;
}

/* For each coordinate c of axis a, the list of real coordinates in its key
 * segment: lists[c * window + n], count[c]. */
static void build_segments(const swo_problem* p, int a, long* lists, int* count) {
    long E = p->extent[a], w = p->window[a];
    for (long c = 0; c < E; c++) {
        int n = 0;
        long lab = segment_label(p, a, c);
        for (long c2 = 0; c2 < E; c2++)
            if (segment_label(p, a, c2) == lab) lists[c * w + n++] = c2;
        count[c] = n;
    }
}

/*
 * Direct-form forward pass.
 * query_index: flat real-token indices ((b*T + t)*H + y)*W + x to evaluate,
 *   or NULL for every real token in order.
 * out: [n_query][heads][head_dim] doubles (for NULL, the full output layout).
 * nthreads: OpenMP threads to use (0: the runtime default).
 * Returns the number of threads used, or a negative value on bad arguments.
 */
int swo_forward(const swo_problem* p, const float* q, const float* k, const float* v,
                const float* table, const long* query_index, long n_query, double* out,
                int nthreads) {
    if (swo_check(p) != 0) return -1;
    const long T = p->extent[0], H = p->extent[1], W = p->extent[2];
    const long tokens = (long)p->batch * T * H * W;
    if (query_index == NULL) n_query = tokens;
    const int heads = p->heads, dim = p->head_dim;
    const long row = (long)heads * dim;
    const int wt = p->window[0], wy = p->window[1], wx = p->window[2];
    const long tdy = 2 * wy - 1, tdx = 2 * wx - 1;
    const long max_keys = (long)wt * wy * wx;

    long* seg[3];
    int* cnt[3];
    for (int a = 0; a < 3; a++) {
        seg[a] = (long*)malloc(sizeof(long) * (size_t)p->extent[a] * p->window[a]);
        cnt[a] = (int*)malloc(sizeof(int) * (size_t)p->extent[a]);
        build_segments(p, a, seg[a], cnt[a]);
    }

    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#endif

#pragma omp parallel
    {
        double* logit = (double*)malloc(sizeof(double) * (size_t)max_keys);
        long* key_tok = (long*)malloc(sizeof(long) * (size_t)max_keys);
        long* key_bias = (long*)malloc(sizeof(long) * (size_t)max_keys);
#pragma omp for schedule(dynamic, 64)
        for (long qi = 0; qi < n_query; qi++) {
            long tok = query_index ? query_index[qi] : qi;
            long x = tok % W, y = (tok / W) % H, t = (tok / (W * H)) % T, b = tok / (W * H * T);
            long lt = swo_local_coord(p, 0, t), ly = swo_local_coord(p, 1, y),
                 lx = swo_local_coord(p, 2, x);
            /* enumerate K(i) as the product of the per-axis segments */
            long nk = 0;
            for (int it = 0; it < cnt[0][t]; it++) {
                long t2 = seg[0][t * wt + it];
                for (int iy = 0; iy < cnt[1][y]; iy++) {
                    long y2 = seg[1][y * wy + iy];
                    for (int ix = 0; ix < cnt[2][x]; ix++) {
                        long x2 = seg[2][x * wx + ix];
                        key_tok[nk] = ((b * T + t2) * H + y2) * W + x2;
                        long dt = lt - swo_local_coord(p, 0, t2) + wt - 1;
                        long dy = ly - swo_local_coord(p, 1, y2) + wy - 1;
                        long dx = lx - swo_local_coord(p, 2, x2) + wx - 1;
                        key_bias[nk] = ((dt * tdy + dy) * tdx + dx) * heads;
                        nk++;
                    }
                }
            }
            for (int h = 0; h < heads; h++) {
                const float* qv = q + tok * row + (long)h * dim;
                double mx = -INFINITY;
                for (long j = 0; j < nk; j++) {
                    const float* kv = k + key_tok[j] * row + (long)h * dim;
                    double dot = 0.0;
                    for (int e = 0; e < dim; e++) dot += (double)qv[e] * (double)kv[e];
                    logit[j] = dot * p->scale + (double)table[key_bias[j] + h];
                    if (logit[j] > mx) mx = logit[j];
                }
                double den = 0.0;
                for (long j = 0; j < nk; j++) {
                    logit[j] = exp(logit[j] - mx);
                    den += logit[j];
                }
                double* o = out + qi * row + (long)h * dim;
                for (int e = 0; e < dim; e++) o[e] = 0.0;
                for (long j = 0; j < nk; j++) {
                    const float* vv = v + key_tok[j] * row + (long)h * dim;
                    double wgt = logit[j] / den;
                    for (int e = 0; e < dim; e++) o[e] += wgt * (double)vv[e];
                }
            }
        }
        free(logit);
        free(key_tok);
        free(key_bias);
    }
    for (int a = 0; a < 3; a++) {
        free(seg[a]);
        free(cnt[a]);
    }
    return used;
}
