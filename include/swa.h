/*
 * swa.h - C ABI of the shifted-window multi-head self-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  The TERRA page ("TERRA: A Hierarchical Parallel Training
 * and Memory Orchestration Framework for High-Resolution AI-based Earth
 * Modeling") describes Earth-forecasting models whose Transformer layers are
 * window-based (Swin) attention with shifted-window execution: tokens of a
 * (time,) latitude, longitude grid leave their spatial layout for a window
 * layout, attend inside windows, and return (abstract; Fig. 5 caption, shift
 * token routes).  Its Table I names the real resolution H, W, the padded
 * resolution H^, W^ and the embedding d; its Table V gives heads N_h and
 * window size w.  The library computes the forward pass of that layer:
 *
 *   for every batch b, head h and real query token i = (t, y, x):
 *     K(i)  = keys sharing i's shifted window, on the same side of the wrap of
 *             every masked axis, excluding pad tokens;
 *     logit = scale * <q_i, k_j> + table[l_t(i)-l_t(j)+w_t-1]
 *                                       [l_y(i)-l_y(j)+w_y-1]
 *                                       [l_x(i)-l_x(j)+w_x-1][h];
 *     o_i   = sum over j in K(i) of softmax_j(logit) * v_j,
 *
 * where the grid is padded at the end of each masked axis, rolled by -shift
 * (rolled[c'] = padded[(c' + s) mod P]), cut into windows, and l_a(c) =
 * ((c - s_a) mod P_a) mod w_a is the position inside the rolled window.
 * Longitude is cyclic (wrapped neighbours attend each other); time and
 * latitude are masked (no attention across the wrap, none to padding).
 *
 * Layouts (all C-contiguous, all device memory):
 *   q, k, v, out : [B][T][H][W][heads][head_dim] over the REAL extents T, H, W,
 *                  element type cfg.dtype (fp32 or bf16);
 *   bias_table   : fp32 [2*w_t-1][2*w_y-1][2*w_x-1][heads];
 *   window-major : [B][nW_t][nW_y][nW_x][N][heads][head_dim], N = w_t*w_y*w_x,
 *                  windows and their tokens in row-major (t, y, x) order of
 *                  the rolled, padded grid; pad slots hold zeros.
 *
 * Ownership.  The caller owns every buffer passed in; they must stay valid
 * until the work queued on the given stream has finished.  A handle owns only
 * its constants and the workspaces it allocates in swa_create and frees in
 * swa_destroy: four window-major tensors for the staged variant, and for the
 * key-blocked schedule a head-major copy of the bias table (heads *
 * table entries floats), which each swa_forward refreshes from bias_table
 * before the attention kernel reads it.  swa_forward never allocates.
 *
 * Errors.  Every call validates its arguments before touching the GPU and
 * returns SWA_ERR_INVALID_ARGUMENT or SWA_ERR_UNSUPPORTED without side
 * effects.  SWA_ERR_HIP means a HIP runtime call or kernel launch failed (for
 * swa_create: no usable gfx950 device); the text of the last failure is
 * available from swa_last_error().  No C++ exception crosses this ABI.
 * All device work is asynchronous on the stream passed in (a hipStream_t;
 * NULL is the default stream).  A handle may be used from one thread at a
 * time; the workspaces are shared by all calls on a handle, so calls on one
 * handle queued on different streams must not overlap.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swa_status {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARGUMENT = 1,
    SWA_ERR_UNSUPPORTED = 2,
    SWA_ERR_OUT_OF_MEMORY = 3,
    SWA_ERR_HIP = 4
} swa_status;

typedef enum swa_dtype {
    SWA_F32 = 0, /* fp32 in and out; fp32 arithmetic throughout */
    SWA_BF16 = 1 /* bf16 in and out; bf16 matrix-core products, fp32 accumulation and softmax */
} swa_dtype;

typedef enum swa_variant {
    SWA_VARIANT_FUSED = 0, /* one kernel: gather and scatter folded into the attention kernel */
    SWA_VARIANT_STAGED = 1 /* gather -> window attention -> scatter, through a window-major workspace */
} swa_variant;

typedef enum swa_schedule {
    SWA_SCHEDULE_AUTO = 0,    /* STREAM when it fits in LDS, else BLOCK, else KEYBLOCK */
    SWA_SCHEDULE_STREAM = 1,  /* bf16: persistent blocks streaming K/V into a two-stage LDS ring */
    SWA_SCHEDULE_BLOCK = 2,   /* bf16: one workgroup per (window, head), windows of up to 512 tokens */
    SWA_SCHEDULE_KEYBLOCK = 3 /* bf16: workgroups of 256 queries of a (window, head) stream K/V in
                                 blocks of 32 keys (online softmax): windows of any size whose
                                 bias slice and token tables leave LDS room for the ring */
} swa_schedule;

typedef enum swa_layer_path {
    SWA_LAYER_AUTO = 0,   /* UNFUSED (the faster path on every shape measured) */
    SWA_LAYER_FUSED = 1,  /* bf16: q, k, v projected per window inside the attention kernel (they never
                             reach device memory), then the output projection GEMM: two launches and a
                             quarter of the workspace */
    SWA_LAYER_UNFUSED = 2 /* projection GEMM, swa_forward, projection GEMM: three launches, q, k, v and
                             the attention output through the workspace */
} swa_layer_path;

typedef struct swa_config {
    int batch;     /* B >= 1 */
    int heads;     /* N_h >= 1 (TERRA, Table V) */
    int head_dim;  /* d / N_h: 32 or 64; 128 with SWA_BF16 (TERRA, Table V: d / N_h = 128) */
    int grid[3];   /* real extents (T, H, W): time, latitude, longitude (TERRA, Table I) */
    int padded[3]; /* padded extents (T^, H^, W^) >= grid; must equal grid on cyclic axes */
    int window[3]; /* window (w_t, w_y, w_x); 1 <= w <= padded, padded % w == 0 */
    int shift[3];  /* shift (s_t, s_y, s_x); 0 <= s < w */
    int cyclic[3]; /* 1: cyclic axis, 0: masked axis.  Usual setting {0, 0, 1} */
    swa_dtype dtype;
    float scale;   /* logit scale, > 0; 0 selects 1/sqrt(head_dim) */
    swa_variant variant;
    swa_schedule schedule; /* bf16 kernel schedule; ignored for SWA_F32 */
    swa_layer_path layer;  /* how swa_layer_forward runs */
} swa_config;

typedef struct swa_handle swa_handle;

/* Derived sizes of a configured handle. */
typedef struct swa_info {
    int64_t windows;            /* B * nW_t * nW_y * nW_x */
    int32_t window_tokens;      /* N = w_t * w_y * w_x */
    int64_t tokens;             /* real tokens B * T * H * W */
    int64_t window_major_elems; /* windows * N * heads * head_dim */
    size_t workspace_bytes;     /* device bytes owned by the handle (staged variant; head-major bias copy of
                                   the key-blocked and per-unit schedules) */
    double nominal_flops;       /* 4 * N^2 * head_dim per (window, head), all windows */
    double algorithmic_bytes;   /* q, k, v read and out written once, real tokens, plus the table */
    int32_t schedule;           /* bf16: the schedule in use (_STREAM, _BLOCK or _KEYBLOCK); fp32: 0 */
    int32_t workgroups;         /* bf16: workgroups per attention launch; fp32: 0 */
    size_t backward_workspace_bytes; /* workspace swa_backward needs; 0: the backward pass does not take
                                        this window (bf16: a bias table slice and token tables past LDS;
                                        fp32: past LDS or head_dim above 64) */
    size_t layer_workspace_bytes;    /* workspace swa_layer_forward needs: q, k, v and the attention
                                        output, tokens * heads * head_dim elements each */
    double layer_flops;              /* swa_layer_forward: 2 * tokens * C * 4C for the two projections
                                        (C = heads * head_dim) plus nominal_flops */
    int32_t backward_schedule;       /* 0: no backward pass; 1: one workgroup per (window, head), the
                                        whole window in LDS (fp32 always); 2: bf16 key-blocked kernels
                                        for windows beyond that (32-token blocks streamed) */
    int32_t layer_path;              /* the path swa_layer_forward takes: SWA_LAYER_FUSED or _UNFUSED */
    int32_t backward_workgroups;     /* bf16 backward schedule 1: workgroups of the persistent kernel
                                        (whole units per workgroup, the next unit's inputs copied
                                        behind the current one); schedule 2 with windows of up to 288
                                        tokens and head_dim 32 or 64: workgroups of the persistent key
                                        kernel (one head, one group of 4 key tiles, a run of windows);
                                        0: one workgroup per (window, head) or query block */
} swa_info;

/*
 * Validates cfg, checks that the current HIP device is a gfx950, and creates
 * a handle.  The workspaces (staged variant; the head-major bias copy of the
 * key-blocked and per-unit schedules) are allocated here.  On failure *out is set to NULL.
 * Errors: INVALID_ARGUMENT (NULL pointers, malformed tiling, unknown enum),
 * UNSUPPORTED (head_dim or window size outside the kernels' range, or an
 * explicit schedule that cannot take the window),
 * HIP (no gfx950 device), OUT_OF_MEMORY (workspace).
 */
swa_status swa_create(const swa_config* cfg, swa_handle** out);

/*
 * The forward pass defined at the top of this header, queued on `stream`.
 * q, k, v, out: device pointers in the layout above, 16-byte aligned; out
 * must not overlap q, k, v or bias_table.  bias_table: device pointer, fp32,
 * 4-byte aligned.  Every real output token is written; nothing else is.
 * Errors: INVALID_ARGUMENT (NULL handle or pointer, misalignment, overlap),
 * HIP (launch failure).
 */
swa_status swa_forward(swa_handle* h, const void* q, const void* k, const void* v,
                       const float* bias_table, void* out, void* stream);

/*
 * swa_forward that also keeps the softmax normaliser of every query for the
 * backward pass (the models are trained: TERRA page, abstract): lse[r * heads
 * + h] = log of the sum of exp(logit) over the keys real token r sees in head
 * h (natural log, the logits of the forward pass above), so that each
 * softmax weight is exp(logit - lse).  lse: device buffer of B*T*H*W*heads
 * fp32 values, 4-byte aligned, owned by the caller, overlapping no other
 * argument; one value per real token and head is written.  out is as
 * swa_forward writes it, bit for bit.  The fused variant only.
 * Errors: as swa_forward; UNSUPPORTED for a staged handle.
 */
swa_status swa_forward_lse(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                           void* out, float* lse, void* stream);

/*
 * Gradients of the forward pass (the pages' models are trained: TERRA page,
 * abstract and Table V).  Given dout = dL/d(out) in the layout of out, writes
 * dq, dk, dv = dL/dq, dL/dk, dL/dv (layout and dtype of q, k, v; every real
 * token) and dtable = dL/d(bias_table) (fp32, the table's layout); all four
 * are overwritten.  The pad tokens of a window have no output, so they add
 * nothing.  workspace: device buffer of info.backward_workspace_bytes bytes,
 * 16-byte aligned, owned by the caller (a head-major copy of the bias table,
 * per-(window, head) shares of the table gradient and their partial sums;
 * with backward_schedule 2 also each query's softmax normaliser and
 * D = rowsum(P * dP); its contents on entry do not matter).  The pass reads and writes the spatial layout whatever the
 * variant and allocates nothing.  backward_schedule 1 (bf16 windows whose
 * Q, K, V, dO and two N x N matrices fit one workgroup's LDS: up to 144
 * tokens with head_dim <= 64, fewer at 128; and fp32): every sum runs in a
 * fixed order, so the results are bitwise reproducible, and the table
 * gradient sums bf16-rounded dS terms in fp32.  backward_schedule 2 (larger
 * bf16 windows): dq, dk, dv are still reproducible; the table gradient sums
 * fp32 dS terms.  Where backward_workgroups > 0 (windows of up to 288 tokens,
 * head_dim 32 or 64) it first sums them over windows per window-local
 * (query, key) pair and then over each entry's pairs, in a fixed order
 * (reproducible); otherwise it sums each window's terms with LDS atomics, in
 * an order that may differ between runs.
 * Asynchronous on `stream`, like swa_forward.
 * Errors: INVALID_ARGUMENT (NULL handle or pointer, misalignment, a buffer
 * written that overlaps another argument), UNSUPPORTED (the window is beyond
 * the backward kernels: backward_workspace_bytes is 0), HIP (launch failure).
 */
swa_status swa_backward(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                        const void* dout, void* dq, void* dk, void* dv, float* dtable, void* workspace,
                        void* stream);

/*
 * swa_backward from the forward pass's output and statistics (out and lse as
 * swa_forward_lse wrote them for the same q, k, v and table; the fused
 * layout): with backward_schedule 2 the query kernel takes each query's
 * softmax normaliser from lse and D = rowsum(dout * out) from out instead of
 * recomputing both in a first pass over the window's keys, so it reads K and
 * V once.  backward_schedule 1 and fp32 form their statistics in LDS as
 * swa_backward does and ignore out and lse: there the results equal
 * swa_backward's bit for bit.  With schedule 2 they differ from it by
 * rounding (out is the bf16-rounded output).  out: 16-byte aligned; lse:
 * 4-byte aligned; both are only read.
 * Errors: as swa_backward; INVALID_ARGUMENT also for NULL out or lse.
 */
swa_status swa_backward_lse(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                            const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* dtable, void* workspace, void* stream);

/*
 * swa_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight training or serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as swa_backward, without the
 * workspace: a head-major copy of the bias table, the per-(window, head)
 * table-gradient shares (and, for backward_schedule 2, the per-query
 * statistics and the per-pair sums) go to a fixed scratch array of 32 MiB in
 * device memory that the library holds on each device it runs on (looked up
 * in swa_create, kept until the process ends).  The windows are processed in
 * passes: of whole chunks of 1/64 of the windows each, as many chunks per
 * pass as the scratch holds, with the table gradient summed chunk by chunk in
 * the order swa_backward sums it; or, where backward_workgroups > 0, of runs
 * of windows sized to the scratch, whose per-pair sums are added to dtable
 * pass by pass.  dq, dk, dv and (with backward_schedule 1) dtable equal
 * swa_backward's bit for bit; otherwise dtable agrees with it to rounding.
 * Queues only
 * kernel launches on `stream` (no allocation, no memset, no host
 * synchronisation).  Every call on one device shares that device's scratch:
 * calls that overlap in time on one device (other streams, other threads,
 * other handles) race and give wrong gradients.  The handle must have been
 * created on the current device.
 * Errors: as swa_backward; also UNSUPPORTED when one pass's smallest layout
 * needs more than the 32 MiB scratch (one chunk of windows: about
 * 2^23 / ((heads * table entries) per window) * 64 windows; swa_backward takes
 * any size), INVALID_ARGUMENT when
 * the current device is not the handle's.
 */
swa_status swa_backward_noalloc(swa_handle* h, const void* q, const void* k, const void* v,
                                const float* bias_table, const void* dout, void* dq, void* dk, void* dv,
                                float* dtable, void* stream);

/*
 * The window attention inside its Swin block's projections (TERRA page,
 * abstract: the models are stacks of Swin blocks; Table V: embedding width
 * d = N_h * head_dim).  With C = heads * head_dim:
 *   qkv = x w_qkv^T + b_qkv;  q, k, v = qkv[.., 0:C], qkv[.., C:2C], qkv[.., 2C:3C]
 *   o   = the forward pass above on q, k, v and bias_table
 *   y   = o w_o^T + b_o
 * Channels are head-major (head h owns channels h*head_dim .. +head_dim-1),
 * so q, k, v and o have exactly the [B][T][H][W][heads][head_dim] layout of
 * swa_forward.  info.layer_path says how it runs: SWA_LAYER_FUSED projects
 * each window's q, k, v head by head inside the attention kernel, so they
 * never reach device memory (bf16; head_dim 32 or 64 with windows of up to
 * 144 tokens, or 128 with up to 80; C a multiple of 32 of at least 96), then runs
 * the output projection; SWA_LAYER_UNFUSED runs three launches.  Both give
 * the same y bit for bit (the fused kernel keeps the projection's operand and
 * reduction order and the attention's arithmetic).  x, y: [B][T][H][W][C] in the handle's dtype.  w_qkv: [3C][C]
 * and w_o: [C][C], the handle's dtype, row-major (a linear layer's
 * [out_features][in_features]).  b_qkv: [3C] and b_o: [C], fp32.  bf16: the
 * products run on bf16 matrix cores with fp32 accumulation; the bias is added
 * in fp32 and q, k, v, o, y are rounded to bf16 once.  x, y, the weights and
 * the workspace are device pointers, 16-byte aligned; biases and table
 * 4-byte aligned.  workspace: info.layer_workspace_bytes bytes, caller-owned;
 * its contents on entry do not matter.  On return it holds o (fused path:
 * tokens * C elements), or q, k, v and o in that order (unfused path: each
 * tokens * C elements).  y must not overlap any other argument, nor the workspace any
 * input.  Asynchronous on `stream`; allocates nothing.
 * Errors: INVALID_ARGUMENT (NULL handle or pointer, misalignment, overlap),
 * UNSUPPORTED (C above 10912: 3C output features exceed the projection's
 * 32768), HIP (launch failure).
 */
swa_status swa_layer_forward(swa_handle* h, const void* x, const void* w_qkv, const float* b_qkv,
                             const float* bias_table, const void* w_o, const float* b_o, void* y,
                             void* workspace, void* stream);

/*
 * The first launch of swa_layer_forward's fused path alone: the attention
 * output o = swa_forward(q, k, v) with q, k, v = x w_qkv^T + b_qkv projected
 * window by window inside the kernel (TERRA page, abstract: Swin blocks).
 * Same x, w_qkv, b_qkv and bias_table as swa_layer_forward; out: [B][T][H][W]
 * [heads][head_dim] in the handle's dtype, 16-byte aligned, every real token
 * written; it must not overlap an input.  Equals the unfused path's o bit for
 * bit.  Asynchronous on `stream`; allocates nothing.
 * Errors: INVALID_ARGUMENT (NULL handle or pointer, misalignment, overlap),
 * UNSUPPORTED (info.layer_path is not SWA_LAYER_FUSED), HIP (launch failure).
 */
swa_status swa_layer_attention(swa_handle* h, const void* x, const void* w_qkv, const float* b_qkv,
                               const float* bias_table, void* out, void* stream);

/*
 * The projection step of swa_layer_forward alone, on any token count:
 *   out[m][n] = sum_k x[m][k] * w[n][k] + bias[n],  m < rows, n < out_features, k < in_features
 * with column n written to d0, d1 or d2 (n / split) at [m][n % split]: the
 * query/key/value projection passes split = C and three tensors, the output
 * projection split = out_features and one tensor (d1, d2 unused, may be
 * NULL).  x [rows][in_features], w [out_features][in_features] and the
 * outputs have element type `dtype` (bf16: bf16 matrix cores, fp32
 * accumulation and bias, one rounding); bias is fp32.  x, w, d0..d2: device
 * pointers, 16-byte aligned; bias 4-byte aligned; the outputs must not
 * overlap the inputs.  Shapes: in_features a positive multiple of 32 up to
 * 65536, out_features and split positive multiples of 8 with
 * out_features <= 3 * split and out_features <= 32768, 0 <= rows < 2^31
 * (rows = 0 does nothing and returns SWA_OK).  Needs a current gfx950 device.  Asynchronous on
 * `stream`; allocates nothing.
 * Errors: INVALID_ARGUMENT (NULL pointer, misalignment, overlap, unknown
 * dtype, negative rows), UNSUPPORTED (shape), HIP (launch failure).
 */
swa_status swa_projection(swa_dtype dtype, const void* x, const void* w, const float* bias, int64_t rows,
                          int32_t out_features, int32_t in_features, int32_t split, void* d0, void* d1,
                          void* d2, void* stream);

/* Frees the handle and its workspace (synchronising the device first when a
 * workspace exists).  NULL is a no-op returning SWA_OK. */
swa_status swa_destroy(swa_handle* h);

/* Sizes derived from the handle's configuration. */
swa_status swa_get_info(const swa_handle* h, swa_info* info);

/* Static text for a status code. */
const char* swa_status_string(swa_status s);

/* Text of the most recent failure on this thread ("" if none). */
const char* swa_last_error(void);

/*
 * The route into the window layout alone (TERRA page, abstract: tokens leave
 * the spatial layout for window layouts; Fig. 5 caption: shift token routes;
 * Table I: the padded resolution H^, W^ the windows tile): pad, roll by
 * -shift, partition.  src [B][T][H][W][heads][head_dim] -> dst window-major
 * (pad slots zeroed).  Same pointer rules as swa_forward; dst holds
 * info.window_major_elems elements.  For tests and for callers that want the
 * window layout itself.
 * Errors: INVALID_ARGUMENT (NULL handle or pointer, misalignment, overlap),
 * HIP (launch failure).
 */
swa_status swa_gather(swa_handle* h, const void* src, void* dst_window_major, void* stream);

/*
 * The route back alone (TERRA page, abstract: tokens return from the window
 * layout to the spatial layout): un-partition, roll by +shift, crop to the
 * real resolution (Table I).  Window-major src -> dst
 * [B][T][H][W][heads][head_dim].  Pad slots of src are not read.
 * Errors: as swa_gather.
 */
swa_status swa_scatter(swa_handle* h, const void* src_window_major, void* dst, void* stream);

/*
 * The attention mask of one window, as the attention kernels evaluate it
 * (TERRA page, abstract: shifted-window execution; Table I: pad tokens of
 * the padded resolution): dev_out[n * N + m] = 1 when key m may be attended
 * by query n of window `window_index` (0 <= window_index < info.windows), that
 * is when neither is pad and they lie on the same side of the wrap of every
 * masked axis, else 0; pad queries get all-zero rows.  dev_out: device buffer
 * of N * N bytes, owned by the caller.
 * Errors: INVALID_ARGUMENT (NULL handle or pointer, window index out of
 * range), HIP (launch failure).
 */
swa_status swa_debug_visibility(swa_handle* h, int64_t window_index, uint8_t* dev_out,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
