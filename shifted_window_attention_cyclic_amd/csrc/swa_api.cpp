// C ABI of the shifted-window attention library: validation, handles,
// variant dispatch and error reporting.  Declarations and the contract of
// every entry point are in include/swa.h.
#include "swa.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>

#include "swa_geometry.h"
#include "swa_layer.h"
#include "swa_projection.h"
#include "swa_backward.h"

struct swa_handle {
    swa_config cfg;
    swa::Geometry g;
    int elem_bytes;
    int device;
    int schedule;       // bf16: SWA_SCHEDULE_STREAM, _BLOCK or _KEYBLOCK; fp32: 0
    int blocks;         // bf16: workgroups per attention launch
    int bwd_blocks;     // workgroups of the persistent backward kernel, 0: one-shot kernels
    int layer_path;     // SWA_LAYER_FUSED or SWA_LAYER_UNFUSED
    size_t wm_bytes;    // bytes of one window-major tensor
    void* workspace;    // staged variant: q, k, v, o window-major tensors
    float* bias_hm;     // key-blocked and per-unit schedules: head-major copy of the bias table
};

// Scratch of swa_backward_noalloc: file-scope device memory, so that the call
// needs no allocation.  Each device holds its own copy from the moment its
// address is first looked up until the process ends.  In host code the name
// stands for a host-side shadow, never a device address: only the address
// hipGetSymbolAddress returns for the current device is passed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices]; // device address of `scratch` on each device, once looked up

swa_status fail(swa_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

swa_status fail_hip(hipError_t e, const char* what) {
    return fail(SWA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Validation that needs no device.  Fills g on success.
swa_status validate(const swa_config* c, swa::Geometry* g, int* elem_bytes) {
    if (c->batch < 1 || c->heads < 1) return fail(SWA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
    if (c->dtype != SWA_F32 && c->dtype != SWA_BF16) return fail(SWA_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (c->variant != SWA_VARIANT_FUSED && c->variant != SWA_VARIANT_STAGED)
        return fail(SWA_ERR_INVALID_ARGUMENT, "unknown variant");
    if (c->schedule != SWA_SCHEDULE_AUTO && c->schedule != SWA_SCHEDULE_STREAM && c->schedule != SWA_SCHEDULE_BLOCK &&
        c->schedule != SWA_SCHEDULE_KEYBLOCK)
        return fail(SWA_ERR_INVALID_ARGUMENT, "unknown schedule");
    if (c->layer != SWA_LAYER_AUTO && c->layer != SWA_LAYER_FUSED && c->layer != SWA_LAYER_UNFUSED)
        return fail(SWA_ERR_INVALID_ARGUMENT, "unknown layer path");
    if (c->head_dim < 1) return fail(SWA_ERR_INVALID_ARGUMENT, "head_dim must be >= 1");
    if (!(isfinite(c->scale)) || c->scale < 0.f)
        return fail(SWA_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
    static const char* axis[3] = {"time", "latitude", "longitude"};
    int64_t tokens = c->batch;
    int N = 1, table = 1;
    int64_t windows = c->batch;
    for (int a = 0; a < 3; a++) {
        char buf[160];
        if (c->grid[a] < 1) {
            snprintf(buf, sizeof buf, "%s extent must be >= 1", axis[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        if (c->cyclic[a] != 0 && c->cyclic[a] != 1) {
            snprintf(buf, sizeof buf, "%s cyclic flag must be 0 or 1", axis[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        if (c->padded[a] < c->grid[a]) {
            snprintf(buf, sizeof buf, "%s padded extent %d is below the extent %d", axis[a], c->padded[a], c->grid[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        if (c->cyclic[a] && c->padded[a] != c->grid[a]) {
            snprintf(buf, sizeof buf, "%s is cyclic and cannot be padded", axis[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        if (c->window[a] < 1 || c->window[a] > c->padded[a]) {
            snprintf(buf, sizeof buf, "%s window %d outside [1, %d]", axis[a], c->window[a], c->padded[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        if (c->padded[a] % c->window[a] != 0) {
            snprintf(buf, sizeof buf, "%s padded extent %d is not a multiple of the window %d", axis[a], c->padded[a], c->window[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        if (c->shift[a] < 0 || c->shift[a] >= c->window[a]) {
            snprintf(buf, sizeof buf, "%s shift %d outside [0, %d)", axis[a], c->shift[a], c->window[a]);
            return fail(SWA_ERR_INVALID_ARGUMENT, buf);
        }
        tokens *= c->grid[a];
        N *= c->window[a];
        table *= 2 * c->window[a] - 1;
        windows *= c->padded[a] / c->window[a];
        if (tokens > (int64_t)1 << 40 || windows > (int64_t)1 << 40)
            return fail(SWA_ERR_UNSUPPORTED, "grid too large");
    }
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
        return fail(SWA_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
    if (c->head_dim == 128 && c->dtype != SWA_BF16)
        return fail(SWA_ERR_UNSUPPORTED, "head_dim 128 needs bf16 (the fp32 kernel takes 32 or 64)");
    if (c->heads > 4096) return fail(SWA_ERR_UNSUPPORTED, "at most 4096 heads");
    if (table >= 1 << 16) return fail(SWA_ERR_UNSUPPORTED, "bias table too large (window too large)");
    const int64_t row = (int64_t)c->heads * c->head_dim;
    // row indices are 32-bit inside the kernels
    if (tokens >= ((int64_t)1 << 31) || windows * N >= ((int64_t)1 << 31))
        return fail(SWA_ERR_UNSUPPORTED, "more than 2^31 tokens");
    if (windows * c->heads >= ((int64_t)1 << 31)) return fail(SWA_ERR_UNSUPPORTED, "too many (window, head) pairs");

    swa::Geometry& G = *g;
    G.batch = c->batch;
    G.heads = c->heads;
    G.head_dim = c->head_dim;
    G.N = N;
    G.nW = 1;
    for (int a = 0; a < 3; a++) {
        G.ext[a] = c->grid[a];
        G.pad[a] = c->padded[a];
        G.win[a] = c->window[a];
        G.shift[a] = c->shift[a];
        G.cyc[a] = c->cyclic[a];
        G.nwin[a] = c->padded[a] / c->window[a];
        G.nW *= G.nwin[a];
    }
    G.windows = windows;
    G.row = (int)row;
    G.tdy = 2 * c->window[1] - 1;
    G.tdx = 2 * c->window[2] - 1;
    G.table_size = table;
    G.c0 = ((c->window[0] - 1) * G.tdy + (c->window[1] - 1)) * G.tdx + (c->window[2] - 1);
    G.scale = c->scale != 0.f ? c->scale : (float)(1.0 / sqrt((double)c->head_dim));
    G.fd_heads = swa::make_fastdiv((uint32_t)c->heads);
    G.fd_nW = swa::make_fastdiv((uint32_t)G.nW);
    G.fd_nwin1 = swa::make_fastdiv((uint32_t)G.nwin[1]);
    G.fd_nwin2 = swa::make_fastdiv((uint32_t)G.nwin[2]);
    G.fd_win1 = swa::make_fastdiv((uint32_t)c->window[1]);
    G.fd_win2 = swa::make_fastdiv((uint32_t)c->window[2]);
    *elem_bytes = c->dtype == SWA_F32 ? 4 : 2;

    if (c->dtype == SWA_BF16) {
        if (!swa::bf16_stream_fits(G, c->variant == SWA_VARIANT_STAGED) && !swa::bf16_block_fits(G) &&
            !swa::bf16_kblock_fits(G))
            return fail(SWA_ERR_UNSUPPORTED, "window too large for the LDS of every bf16 schedule");
    } else if (swa::attention_lds_bytes(G, false, false) > 160 * 1024) {
        return fail(SWA_ERR_UNSUPPORTED, "window too large for the LDS of one workgroup");
    }
    return SWA_OK;
}

// The device address of `scratch` on device dev, which must be current; looked
// up once per device.
swa_status scratch_for_device(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(SWA_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(SWA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SWA_OK;
}

size_t io_bytes(const swa_handle* h) {
    return (size_t)h->g.batch * h->g.ext[0] * h->g.ext[1] * h->g.ext[2] * h->g.row * h->elem_bytes;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

} // namespace

extern "C" {

const char* swa_status_string(swa_status s) {
    switch (s) {
    case SWA_OK: return "ok";
    case SWA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SWA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SWA_ERR_OUT_OF_MEMORY: return "out of device memory";
    case SWA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* swa_last_error(void) { return g_last_error.c_str(); }

swa_status swa_create(const swa_config* cfg, swa_handle** out) {
    if (out) *out = nullptr;
    if (!cfg || !out) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    swa::Geometry g;
    int eb = 0;
    swa_status st = validate(cfg, &g, &eb);
    if (st != SWA_OK) return st;

    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(SWA_ERR_HIP, "no HIP device");
    }
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail_hip(e, "hipGetDevice");
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(SWA_ERR_HIP, std::string("device is ") + prop.gcnArchName + ", kernels are built for gfx950");
    // LDS a workgroup may use: gfx950 has 160 KB per CU
    int optin = 0, per_cu = 0;
    (void)hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev);
    (void)hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    (void)hipGetLastError();
    int max_lds = optin > per_cu ? optin : per_cu;
    if (max_lds < 64 * 1024) max_lds = 64 * 1024;
    if (max_lds > 160 * 1024) max_lds = 160 * 1024;
    const bool staged = cfg->variant == SWA_VARIANT_STAGED;
    const size_t need = swa::attention_lds_bytes(g, cfg->dtype == SWA_BF16, staged);
    if (need > (size_t)max_lds) {
        char buf[160];
        snprintf(buf, sizeof buf, "window needs %zu bytes of LDS, the device allows %d", need, max_lds);
        return fail(SWA_ERR_UNSUPPORTED, buf);
    }
    if ((e = swa::prepare_kernels(max_lds)) != hipSuccess) return fail_hip(e, "hipFuncSetAttribute");
    {
        // set-up of swa_backward_noalloc on this device (once per device)
        void* sp = nullptr;
        const swa_status ss = scratch_for_device(dev, &sp);
        if (ss != SWA_OK) return ss;
    }
    if ((e = swa::prepare_backward_kernels(max_lds)) != hipSuccess) return fail_hip(e, "hipFuncSetAttribute");
    if ((e = swa::prepare_layer_kernels(max_lds)) != hipSuccess) return fail_hip(e, "hipFuncSetAttribute");
    const bool fused_layer = cfg->dtype == SWA_BF16 && swa::layer_fused_fits(g);
    if (cfg->layer == SWA_LAYER_FUSED && !fused_layer)
        return fail(SWA_ERR_UNSUPPORTED, "the fused layer kernel does not take this problem");
    int schedule = 0, blocks = 0;
    if (cfg->dtype == SWA_BF16) {
        // AUTO: the streaming schedule, else the per-unit one, else the key-blocked one,
        // each only when its workgroup fits and can be resident
        const bool fit[4] = {false, swa::bf16_stream_fits(g, staged), swa::bf16_block_fits(g),
                             swa::bf16_kblock_fits(g)};
        const int order[3] = {SWA_SCHEDULE_STREAM, SWA_SCHEDULE_BLOCK, SWA_SCHEDULE_KEYBLOCK};
        for (int sc : order) {
            if (cfg->schedule != SWA_SCHEDULE_AUTO && cfg->schedule != sc) continue;
            if (!fit[sc]) {
                if (cfg->schedule == sc) return fail(SWA_ERR_UNSUPPORTED, "the requested schedule cannot take this window");
                continue;
            }
            e = sc == SWA_SCHEDULE_KEYBLOCK ? swa::kblock_plan(g, &blocks)
                                            : swa::bf16_plan(g, sc == SWA_SCHEDULE_STREAM, &blocks);
            if (e != hipSuccess) return fail_hip(e, "occupancy query");
            if (blocks >= 1) {
                schedule = sc;
                break;
            }
        }
        if (schedule == 0) return fail(SWA_ERR_UNSUPPORTED, "attention kernel does not fit on a compute unit");
    }
    int bwd_blocks = 0;
    if ((e = swa::backward_plan(g, cfg->dtype == SWA_BF16, &bwd_blocks)) != hipSuccess)
        return fail_hip(e, "occupancy query");

    swa_handle* h = new (std::nothrow) swa_handle();
    if (!h) return fail(SWA_ERR_OUT_OF_MEMORY, "host allocation");
    h->cfg = *cfg;
    h->g = g;
    h->elem_bytes = eb;
    h->device = dev;
    h->schedule = schedule;
    h->blocks = blocks;
    h->bwd_blocks = bwd_blocks;
    // AUTO takes the unfused layer: it is the faster one on every measured shape
    h->layer_path = fused_layer && cfg->layer == SWA_LAYER_FUSED ? SWA_LAYER_FUSED : SWA_LAYER_UNFUSED;
    h->wm_bytes = (size_t)g.windows * g.N * g.row * eb;
    h->workspace = nullptr;
    h->bias_hm = nullptr;
    if (cfg->variant == SWA_VARIANT_STAGED) {
        e = hipMalloc(&h->workspace, 4 * h->wm_bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            delete h;
            return fail(SWA_ERR_OUT_OF_MEMORY, "staged workspace");
        }
    }
    if (schedule == SWA_SCHEDULE_KEYBLOCK || schedule == SWA_SCHEDULE_BLOCK) {
        e = hipMalloc((void**)&h->bias_hm, swa::bf16_kblock_workspace_bytes(g));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            if (h->workspace) (void)hipFree(h->workspace);
            delete h;
            return fail(SWA_ERR_OUT_OF_MEMORY, "bias table copy");
        }
    }
    *out = h;
    return SWA_OK;
}

swa_status swa_destroy(swa_handle* h) {
    if (!h) return SWA_OK;
    swa_status st = SWA_OK;
    if (h->workspace || h->bias_hm) {
        hipError_t e = hipDeviceSynchronize();
        if (e == hipSuccess && h->workspace) e = hipFree(h->workspace);
        if (e == hipSuccess && h->bias_hm) e = hipFree(h->bias_hm);
        if (e != hipSuccess) st = fail_hip(e, "releasing the workspace");
    }
    delete h;
    return st;
}

swa_status swa_get_info(const swa_handle* h, swa_info* info) {
    if (!h || !info) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    const swa::Geometry& g = h->g;
    info->windows = g.windows;
    info->window_tokens = g.N;
    info->tokens = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    info->window_major_elems = g.windows * g.N * (int64_t)g.row;
    info->workspace_bytes = (h->workspace ? 4 * h->wm_bytes : 0) +
                            (h->bias_hm ? swa::bf16_kblock_workspace_bytes(g) : 0);
    info->nominal_flops = 4.0 * g.N * (double)g.N * g.head_dim * (double)g.windows * g.heads;
    info->algorithmic_bytes = 4.0 * (double)info->tokens * g.row * h->elem_bytes + 4.0 * g.table_size * g.heads;
    const bool bf16 = h->cfg.dtype == SWA_BF16;
    info->schedule = bf16 ? h->schedule : 0;
    info->workgroups = bf16 ? h->blocks : 0;
    info->backward_workspace_bytes = swa::backward_fits(g, bf16) ? swa::backward_workspace_bytes(g) : 0;
    info->backward_schedule = swa::backward_schedule(g, bf16);
    info->backward_workgroups = h->bwd_blocks;
    info->layer_path = h->layer_path;
    info->layer_workspace_bytes = (h->layer_path == SWA_LAYER_FUSED ? 1 : 4) * io_bytes(h);
    info->layer_flops = 8.0 * (double)info->tokens * g.row * (double)g.row + info->nominal_flops;
    return SWA_OK;
}

// The forward pass after argument checks; lse (fused variant only) may be null.
static swa_status forward(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                          void* out, float* lse, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const swa::Geometry& g = h->g;
    const bool bf16 = h->cfg.dtype == SWA_BF16;
    hipError_t e;
    auto attention = [&](bool staged, const void* aq, const void* ak, const void* av, void* ao) {
        if (!bf16)
            return swa::launch_attention_f32(g, staged, (const float*)aq, (const float*)ak, (const float*)av,
                                             bias_table, (float*)ao, lse, s);
        if (h->schedule == SWA_SCHEDULE_KEYBLOCK)
            return swa::launch_attention_kblock(g, staged, (const uint16_t*)aq, (const uint16_t*)ak,
                                                (const uint16_t*)av, bias_table, h->bias_hm, (uint16_t*)ao, lse, s);
        return swa::launch_attention_bf16(g, h->schedule == SWA_SCHEDULE_STREAM, h->blocks, staged,
                                          (const uint16_t*)aq, (const uint16_t*)ak, (const uint16_t*)av, bias_table,
                                          h->bias_hm, (uint16_t*)ao, lse, s);
    };
    if (h->cfg.variant == SWA_VARIANT_FUSED) {
        e = attention(false, q, k, v, out);
        return e == hipSuccess ? SWA_OK : fail_hip(e, "attention launch");
    }
    char* ws = (char*)h->workspace;
    void* wq = ws;
    void* wk = ws + h->wm_bytes;
    void* wv = ws + 2 * h->wm_bytes;
    void* wo = ws + 3 * h->wm_bytes;
    if ((e = swa::launch_gather(g, h->elem_bytes, q, wq, s)) != hipSuccess) return fail_hip(e, "gather launch");
    if ((e = swa::launch_gather(g, h->elem_bytes, k, wk, s)) != hipSuccess) return fail_hip(e, "gather launch");
    if ((e = swa::launch_gather(g, h->elem_bytes, v, wv, s)) != hipSuccess) return fail_hip(e, "gather launch");
    if ((e = attention(true, wq, wk, wv, wo)) != hipSuccess) return fail_hip(e, "attention launch");
    if ((e = swa::launch_scatter(g, h->elem_bytes, wo, out, s)) != hipSuccess) return fail_hip(e, "scatter launch");
    return SWA_OK;
}

static swa_status forward_args(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                               void* out) {
    if (!h || !q || !k || !v || !bias_table || !out) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(bias_table, 4))
        return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer (q, k, v, out need 16 bytes)");
    const size_t n = io_bytes(h);
    const size_t nt = (size_t)h->g.table_size * h->g.heads * sizeof(float);
    if (overlap(out, n, q, n) || overlap(out, n, k, n) || overlap(out, n, v, n) || overlap(out, n, bias_table, nt))
        return fail(SWA_ERR_INVALID_ARGUMENT, "out overlaps an input");
    return SWA_OK;
}

// bytes of a log-sum-exp tensor: one float per real token and head
static size_t lse_bytes(const swa_handle* h) {
    const swa::Geometry& g = h->g;
    return (size_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2] * g.heads * sizeof(float);
}

swa_status swa_forward(swa_handle* h, const void* q, const void* k, const void* v,
                       const float* bias_table, void* out, void* stream) {
    const swa_status st = forward_args(h, q, k, v, bias_table, out);
    return st != SWA_OK ? st : forward(h, q, k, v, bias_table, out, nullptr, stream);
}

swa_status swa_forward_lse(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                           void* out, float* lse, void* stream) {
    swa_status st = forward_args(h, q, k, v, bias_table, out);
    if (st != SWA_OK) return st;
    if (!lse) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(lse, 4)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned lse");
    if (h->cfg.variant != SWA_VARIANT_FUSED)
        return fail(SWA_ERR_UNSUPPORTED, "the statistics come with the fused variant only");
    const size_t n = io_bytes(h);
    const size_t nt = (size_t)h->g.table_size * h->g.heads * sizeof(float);
    const size_t nl = lse_bytes(h);
    if (overlap(lse, nl, q, n) || overlap(lse, nl, k, n) || overlap(lse, nl, v, n) || overlap(lse, nl, out, n) ||
        overlap(lse, nl, bias_table, nt))
        return fail(SWA_ERR_INVALID_ARGUMENT, "lse overlaps another argument");
    return forward(h, q, k, v, bias_table, out, lse, stream);
}

// Argument checks of the backward passes and the launch; o and lse (the
// forward's output and statistics) may both be null.
static swa_status backward(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dtable, void* workspace, void* stream) {
    if (!h || !q || !k || !v || !bias_table || !dout || !dq || !dk || !dv || !dtable || !workspace)
        return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    const void* tensors[] = {q, k, v, dout, dq, dk, dv, workspace};
    for (const void* p : tensors)
        if (!aligned(p, 16)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer (tensors and workspace need 16 bytes)");
    if (!aligned(bias_table, 4) || !aligned(dtable, 4)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned table");
    if ((o && !aligned(o, 16)) || (lse && !aligned(lse, 4)))
        return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned out or lse");
    const swa::Geometry& g = h->g;
    const bool bf16 = h->cfg.dtype == SWA_BF16;
    if (!swa::backward_fits(g, bf16))
        return fail(SWA_ERR_UNSUPPORTED, "the backward kernels do not take this window");
    const size_t n = io_bytes(h);
    const size_t nt = (size_t)g.table_size * g.heads * sizeof(float);
    const size_t nw = swa::backward_workspace_bytes(g);
    const size_t nl = lse_bytes(h);
    // every buffer written must be disjoint from every other argument
    const void* all[] = {q, k, v, dout, bias_table, o, lse, dq, dk, dv, dtable, workspace};
    const size_t len[] = {n, n, n, n, nt, o ? n : 0, lse ? nl : 0, n, n, n, nt, nw};
    for (int i = 7; i < 12; i++)
        for (int j = 0; j < 12; j++)
            if (j != i && all[j] && overlap(all[i], len[i], all[j], len[j]))
                return fail(SWA_ERR_INVALID_ARGUMENT, "a gradient or the workspace overlaps another argument");
    hipError_t e = swa::launch_backward(g, bf16, q, k, v, bias_table, dout, dq, dk, dv, dtable, workspace, o, lse,
                                        h->bwd_blocks, (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "backward launch");
}

swa_status swa_backward(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                        const void* dout, void* dq, void* dk, void* dv, float* dtable, void* workspace,
                        void* stream) {
    return backward(h, q, k, v, bias_table, nullptr, nullptr, dout, dq, dk, dv, dtable, workspace, stream);
}

swa_status swa_backward_lse(swa_handle* h, const void* q, const void* k, const void* v, const float* bias_table,
                            const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* dtable, void* workspace, void* stream) {
    if (!out || !lse) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    return backward(h, q, k, v, bias_table, out, lse, dout, dq, dk, dv, dtable, workspace, stream);
}

swa_status swa_backward_noalloc(swa_handle* h, const void* q, const void* k, const void* v,
                                const float* bias_table, const void* dout, void* dq, void* dk, void* dv,
                                float* dtable, void* stream) {
    if (!h || !q || !k || !v || !bias_table || !dout || !dq || !dk || !dv || !dtable)
        return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    const void* tensors[] = {q, k, v, dout, dq, dk, dv};
    for (const void* p : tensors)
        if (!aligned(p, 16)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer (tensors need 16 bytes)");
    if (!aligned(bias_table, 4) || !aligned(dtable, 4)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned table");
    const swa::Geometry& g = h->g;
    const bool bf16 = h->cfg.dtype == SWA_BF16;
    if (!swa::backward_fits(g, bf16))
        return fail(SWA_ERR_UNSUPPORTED, "the backward kernels do not take this window");
    const size_t need = swa::backward_scratch_bytes(g, bf16);
    if (need > kScratchBytes) {
        char buf[200];
        snprintf(buf, sizeof buf,
                 "one chunk of windows needs %zu bytes of scratch, above the %zu of swa_backward_noalloc "
                 "(swa_backward takes a workspace of any size)", need, kScratchBytes);
        return fail(SWA_ERR_UNSUPPORTED, buf);
    }
    const size_t n = io_bytes(h);
    const size_t nt = (size_t)g.table_size * g.heads * sizeof(float);
    const void* all[] = {q, k, v, dout, bias_table, dq, dk, dv, dtable};
    const size_t len[] = {n, n, n, n, nt, n, n, n, nt};
    for (int i = 5; i < 9; i++)
        for (int j = 0; j < 9; j++)
            if (j != i && overlap(all[i], len[i], all[j], len[j]))
                return fail(SWA_ERR_INVALID_ARGUMENT, "a gradient overlaps another argument");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev != h->device) return fail(SWA_ERR_INVALID_ARGUMENT, "the handle was created on another device");
    void* sp = nullptr;
    const swa_status st = scratch_for_device(dev, &sp); // looked up in swa_create: no runtime call here
    if (st != SWA_OK) return st;
    e = swa::launch_backward_scratch(g, bf16, q, k, v, bias_table, dout, dq, dk, dv, dtable, sp, kScratchBytes,
                                     h->bwd_blocks, (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "backward launch");
}

swa_status swa_layer_forward(swa_handle* h, const void* x, const void* w_qkv, const float* b_qkv,
                             const float* bias_table, const void* w_o, const float* b_o, void* y,
                             void* workspace, void* stream) {
    if (!h || !x || !w_qkv || !b_qkv || !bias_table || !w_o || !b_o || !y || !workspace)
        return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    const void* wide[] = {x, w_qkv, w_o, y, workspace};
    for (const void* p : wide)
        if (!aligned(p, 16)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer (x, y, weights and workspace need 16 bytes)");
    if (!aligned(b_qkv, 4) || !aligned(b_o, 4) || !aligned(bias_table, 4))
        return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned bias or table");
    const swa::Geometry& g = h->g;
    const int C = g.row;
    const int64_t M = (int64_t)g.batch * g.ext[0] * g.ext[1] * g.ext[2];
    if (!swa::projection_fits(M, 3 * C, C, C)) return fail(SWA_ERR_UNSUPPORTED, "projection shape");
    const size_t n = io_bytes(h);
    const size_t eb = h->elem_bytes;
    const size_t nt = (size_t)g.table_size * g.heads * sizeof(float);
    // y is disjoint from every other argument; the workspace from every input
    const void* all[] = {x, w_qkv, b_qkv, bias_table, w_o, b_o, y, workspace};
    const size_t nws = (h->layer_path == SWA_LAYER_FUSED ? 1 : 4) * n;
    const size_t len[] = {n, 3 * (size_t)C * C * eb, 3 * (size_t)C * 4, nt, (size_t)C * C * eb, (size_t)C * 4, n,
                          nws};
    for (int i = 6; i < 8; i++)
        for (int j = 0; j < 8; j++)
            if (j != i && overlap(all[i], len[i], all[j], len[j]))
                return fail(SWA_ERR_INVALID_ARGUMENT, "y or the workspace overlaps another argument");
    hipStream_t s = (hipStream_t)stream;
    const bool bf16 = h->cfg.dtype == SWA_BF16;
    if (h->layer_path == SWA_LAYER_FUSED) {
        // q, k, v projected inside the attention kernel; o through the workspace
        hipError_t e = swa::launch_layer_qkv_attention(g, (const uint16_t*)x, (const uint16_t*)w_qkv, b_qkv,
                                                       bias_table, (uint16_t*)workspace, s);
        if (e != hipSuccess) return fail_hip(e, "fused layer launch");
        e = swa::launch_projection(true, workspace, w_o, b_o, M, C, C, C, y, y, y, s);
        return e == hipSuccess ? SWA_OK : fail_hip(e, "projection launch");
    }
    char* ws = (char*)workspace;
    void* q = ws;
    void* k = ws + n;
    void* v = ws + 2 * n;
    void* o = ws + 3 * n;
    hipError_t e = swa::launch_projection(bf16, x, w_qkv, b_qkv, M, 3 * C, C, C, q, k, v, s);
    if (e != hipSuccess) return fail_hip(e, "projection launch");
    swa_status st = swa_forward(h, q, k, v, bias_table, o, stream);
    if (st != SWA_OK) return st;
    e = swa::launch_projection(bf16, o, w_o, b_o, M, C, C, C, y, y, y, s);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "projection launch");
}

swa_status swa_layer_attention(swa_handle* h, const void* x, const void* w_qkv, const float* b_qkv,
                               const float* bias_table, void* out, void* stream) {
    if (!h || !x || !w_qkv || !b_qkv || !bias_table || !out) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(x, 16) || !aligned(w_qkv, 16) || !aligned(out, 16) || !aligned(b_qkv, 4) || !aligned(bias_table, 4))
        return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer (x, w_qkv and out need 16 bytes)");
    if (h->layer_path != SWA_LAYER_FUSED) return fail(SWA_ERR_UNSUPPORTED, "the handle's layer path is not fused");
    const swa::Geometry& g = h->g;
    const int C = g.row;
    const size_t n = io_bytes(h);
    const size_t nt = (size_t)g.table_size * g.heads * sizeof(float);
    const void* ins[] = {x, w_qkv, b_qkv, bias_table};
    const size_t len[] = {n, 3 * (size_t)C * C * 2, 3 * (size_t)C * 4, nt};
    for (int j = 0; j < 4; j++)
        if (overlap(out, n, ins[j], len[j])) return fail(SWA_ERR_INVALID_ARGUMENT, "out overlaps an input");
    const hipError_t e = swa::launch_layer_qkv_attention(g, (const uint16_t*)x, (const uint16_t*)w_qkv, b_qkv,
                                                         bias_table, (uint16_t*)out, (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "fused layer launch");
}

swa_status swa_projection(swa_dtype dtype, const void* x, const void* w, const float* bias, int64_t rows,
                          int32_t out_features, int32_t in_features, int32_t split, void* d0, void* d1,
                          void* d2, void* stream) {
    if (dtype != SWA_F32 && dtype != SWA_BF16) return fail(SWA_ERR_INVALID_ARGUMENT, "unknown dtype");
    const int nt = split > 0 ? (out_features + split - 1) / split : 0;
    if (!x || !w || !bias || !d0 || (nt > 1 && !d1) || (nt > 2 && !d2))
        return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (rows < 0) return fail(SWA_ERR_INVALID_ARGUMENT, "negative row count");
    if (!swa::projection_fits(rows > 0 ? rows : 1, out_features, in_features, split))
        return fail(SWA_ERR_UNSUPPORTED, "projection shape (in_features a multiple of 32 up to 65536, out_features "
                                         "and split multiples of 8, out_features <= 3 * split and <= 32768, rows "
                                         "below 2^31)");
    if (rows == 0) return SWA_OK;
    void* dst[3] = {d0, nt > 1 ? d1 : d0, nt > 2 ? d2 : d0};
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(bias, 4))
        return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer (x, w and outputs need 16 bytes)");
    const size_t eb = dtype == SWA_F32 ? 4 : 2;
    const size_t nx = (size_t)rows * in_features * eb, nw = (size_t)out_features * in_features * eb;
    const size_t nb = (size_t)out_features * 4;
    for (int t = 0; t < nt; t++) {
        const int cols = out_features - t * split < split ? out_features - t * split : split;
        const size_t nd = ((size_t)(rows - 1) * split + cols) * eb;
        if (!aligned(dst[t], 16)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned output");
        if (overlap(dst[t], nd, x, nx) || overlap(dst[t], nd, w, nw) || overlap(dst[t], nd, bias, nb))
            return fail(SWA_ERR_INVALID_ARGUMENT, "an output overlaps an input");
    }
    hipError_t e = swa::launch_projection(dtype == SWA_BF16, x, w, bias, rows, out_features, in_features, split,
                                          dst[0], dst[1], dst[2], (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "projection launch");
}

swa_status swa_gather(swa_handle* h, const void* src, void* dst_window_major, void* stream) {
    if (!h || !src || !dst_window_major) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(src, 16) || !aligned(dst_window_major, 16)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer");
    if (overlap(src, io_bytes(h), dst_window_major, h->wm_bytes))
        return fail(SWA_ERR_INVALID_ARGUMENT, "dst overlaps src");
    hipError_t e = swa::launch_gather(h->g, h->elem_bytes, src, dst_window_major, (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "gather launch");
}

swa_status swa_scatter(swa_handle* h, const void* src_window_major, void* dst, void* stream) {
    if (!h || !src_window_major || !dst) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!aligned(src_window_major, 16) || !aligned(dst, 16)) return fail(SWA_ERR_INVALID_ARGUMENT, "misaligned pointer");
    if (overlap(dst, io_bytes(h), src_window_major, h->wm_bytes))
        return fail(SWA_ERR_INVALID_ARGUMENT, "dst overlaps src");
    hipError_t e = swa::launch_scatter(h->g, h->elem_bytes, src_window_major, dst, (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "scatter launch");
}

swa_status swa_debug_visibility(swa_handle* h, int64_t window_index, uint8_t* dev_out, void* stream) {
    if (!h || !dev_out) return fail(SWA_ERR_INVALID_ARGUMENT, "NULL argument");
    if (window_index < 0 || window_index >= h->g.windows) return fail(SWA_ERR_INVALID_ARGUMENT, "window index out of range");
    hipError_t e = swa::launch_visibility(h->g, window_index, dev_out, (hipStream_t)stream);
    return e == hipSuccess ? SWA_OK : fail_hip(e, "visibility launch");
}

} // extern "C"
