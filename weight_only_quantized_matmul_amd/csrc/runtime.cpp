// libwqmm runtime: device table, resident tensors, groups, dispatch and the
// C ABI declared in include/wqmm.h.
//
// Shape of the contract (colibri-analysis "CUDA 后端", section 1): a
// self-contained extern "C" library that opens devices, reports memory,
// uploads a quantized [O, I] tensor once (re-uploads only validate), runs the
// matmul and frees tensors; every GPU failure is reported to the caller, who
// may fall back to the CPU (same page, section 3.1). Startup problems (no
// device, bad ordinals) are errors, not a silent CPU mode (colibri docs
// "CUDA backend (Linux)", introduction).
#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <mutex>
#include <new>

#include "skinny_group.h"
#include "staging.h"
#include "wq_internal.h"

namespace {

// Device scratch of wq_matmul_dev_noalloc (the tiled path's activation
// planes and split-K partials), for callers that cannot allocate. One copy
// per device, held until the process ends. In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device in wq_init (DeviceCtx::scratch) and only that address
// is passed on.
constexpr size_t kScratchBytes = (size_t)WQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceCtx {
    bool open = false;
    uint16_t *scratch = nullptr;   // device address of this device's `scratch`
    hipStream_t stream = nullptr;  // library stream for the host-pointer calls
    int cus = 0;
    size_t total_mem = 0;
    char name[256] = {0};
    char arch[64] = {0};
    float *d_x = nullptr;
    size_t x_cap = 0;  // bytes
    float *d_y = nullptr;
    size_t y_cap = 0;  // bytes
    // pinned host staging of the host-pointer calls, mapped into the
    // device's address space (dh_*: its device addresses), read and written
    // by copy kernels on the library stream
    float *h_x = nullptr, *dh_x = nullptr;
    size_t hx_cap = 0;  // bytes
    float *h_y = nullptr, *dh_y = nullptr;
    size_t hy_cap = 0;  // bytes
    // Tiled workspaces (activation planes, split-K partials, the gated
    // intermediate), one per stream that ran such a call, so calls on
    // different streams may overlap. At most kStreamWorkspaces per device;
    // a new stream beyond that takes over the least recently used one.
    struct StreamWs {
        hipStream_t st = nullptr;
        bool live = false;
        uint16_t *p = nullptr;
        size_t cap = 0;  // bytes
        unsigned long long last = 0;
    };
    static constexpr int kStreamWorkspaces = 8;
    StreamWs ws[kStreamWorkspaces];
    unsigned long long ws_clock = 0;
    size_t lib_bytes = 0;      // device bytes held by tensors, groups and the workspace
    std::recursive_mutex mu;
};

struct Config {
    int force_path = 0;  // 0 auto, 1 gemv, 2 tiled, 3 skinny
    int gemv_max_s = -1;  // -1: per-format default (gemv_limit); else WQ_GEMV_MAX_S
    long long mem_limit = 0;  // 0: none
    int fault = 0;            // 0 none, 1 upload, 2 launch
    int verbose = 0;
    int waves_per_cu = 0;  // 0: per kernel shape (GEMV) / 8 (grouped launches)
    int tiled_mode = wq::kTiledBF16X3;  // quantized weights: exact bf16 split of x
    int tiled_shape = 0;                // 0: by size; else bm * 1000000 + bn * 1000 + bk
    int skinny_ring = 0;                // 0: default; else chunks of loads in flight (2, 4, 6)
};

DeviceCtx g_dev[WQ_MAX_DEVICES];
Config g_cfg;
std::mutex g_init_mu;

constexpr int kDefaultCUs = 256;  // MI355X; used by the host-only plan description

void read_env(Config &c) {
    c = Config();
    if (const char *v = getenv("WQ_FORCE_PATH")) {
        if (!strcmp(v, "gemv")) c.force_path = 1;
        else if (!strcmp(v, "tiled")) c.force_path = 2;
        else if (!strcmp(v, "skinny")) c.force_path = 3;
    }
    if (const char *v = getenv("WQ_GEMV_MAX_S")) {
        int n = atoi(v);
        if (n >= 0 && n <= 8) c.gemv_max_s = n;
    }
    if (const char *v = getenv("WQ_MEM_LIMIT_BYTES")) c.mem_limit = atoll(v);
    if (const char *v = getenv("WQ_FAULT")) {
        if (!strcmp(v, "upload")) c.fault = 1;
        else if (!strcmp(v, "launch")) c.fault = 2;
    }
    if (const char *v = getenv("WQ_VERBOSE")) c.verbose = atoi(v);
    if (const char *v = getenv("WQ_TILED_MODE")) {
        if (!strcmp(v, "fp32")) c.tiled_mode = wq::kTiledF32;
        else if (!strcmp(v, "bf16x3")) c.tiled_mode = wq::kTiledBF16X3;
        else if (!strcmp(v, "bf16")) c.tiled_mode = wq::kTiledBF16;
    }
    if (const char *v = getenv("WQ_TILED_SHAPE")) {
        int bm = 0, bn = 0, bk = 0;
        if (sscanf(v, "%dx%dx%d", &bm, &bn, &bk) == 3) c.tiled_shape = bm * 1000000 + bn * 1000 + bk;
    }
    if (const char *v = getenv("WQ_SKINNY_RING")) c.skinny_ring = atoi(v);
    if (const char *v = getenv("WQ_WAVES_PER_CU")) {
        int n = atoi(v);
        if (n >= 1 && n <= 32) c.waves_per_cu = n;
    }
}

// Makes `dev` current for the scope, restoring the caller's device after.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
            switched = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (switched) (void)hipSetDevice(prev);
    }
};

bool valid_fmt(int fmt) { return fmt >= WQ_F32 && fmt <= WQ_I2; }

bool tensor_ok(const wq_tensor *t) { return t != nullptr && t->magic == wq::kTensorMagic; }

bool device_open(int dev) { return dev >= 0 && dev < WQ_MAX_DEVICES && g_dev[dev].open; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return WQ_OK;
    if (e == hipErrorOutOfMemory) return WQ_E_OOM;
    return WQ_E_HIP;
}

int dev_alloc(DeviceCtx &d, void **p, size_t bytes) {
    if (g_cfg.mem_limit > 0 && (long long)(d.lib_bytes + bytes) > g_cfg.mem_limit) return WQ_E_OOM;
    if (hipMalloc(p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        return WQ_E_OOM;
    }
    d.lib_bytes += bytes;
    return WQ_OK;
}

void dev_free(DeviceCtx &d, void *p, size_t bytes) {
    if (p) {
        (void)hipFree(p);
        d.lib_bytes -= std::min(d.lib_bytes, bytes);
    }
}

// Largest S served by the register GEMV for one tensor: one activation
// row for the quantized formats (from two rows on, the vector ALUs run S
// FMAs per weight element while the matrix-core kernel for few rows spends
// about two instructions per element on the decode alone); f32 weights keep
// the GEMV up to S = 8.
int gemv_limit(int fmt) {
    if (g_cfg.gemv_max_s >= 0) return g_cfg.gemv_max_s;
    return fmt == WQ_F32 ? WQ_GEMV_MAX_S : 1;
}

// Largest S for which a group runs as one grouped GEMV launch (above it,
// one call per tensor): the grouped launch keeps the register GEMV up to
// S = 4 for int4 / int2 and S = 8 otherwise.
int group_gemv_limit(int fmt) {
    if (g_cfg.gemv_max_s >= 0) return g_cfg.gemv_max_s;
    return (fmt == WQ_I4 || fmt == WQ_I2) ? 4 : WQ_GEMV_MAX_S;
}

// Which path a call takes: 1 (register GEMV), 2 (tiled), 3 (matrix-core
// kernel for few rows). x_vec: x is 16-byte aligned (the few-rows kernel
// reads it in 16-byte runs and also needs I % 4 == 0).
// Group-scaled tensors (gs) never take the few-rows kernel.
int choose_path(int fmt, int O, int I, int S, int cus, wq::GemvPlan *gp, int gs = 0, bool x_vec = true,
                wq::SkinnyPlan *sp = nullptr) {
    auto skinny_ok = [&]() {
        if (!x_vec) return false;
        const wq::SkinnyPlan p = wq::plan_skinny(fmt, O, I, S, cus, g_cfg.skinny_ring, gs);
        if (sp) *sp = p;
        return p.ok;
    };
    if (g_cfg.force_path == 3 && skinny_ok()) return 3;
    if (g_cfg.force_path != 2 && g_cfg.force_path != 3 && S <= gemv_limit(fmt)) {
        *gp = wq::plan_gemv(fmt, O, I, S, cus, g_cfg.waves_per_cu);
        if (gp->ok) return 1;
    }
    if (g_cfg.force_path == 1) {
        *gp = wq::plan_gemv(fmt, O, I, S, cus, g_cfg.waves_per_cu);
        if (gp->ok) return 1;
    }
    if (g_cfg.force_path == 0 && skinny_ok()) return 3;
    // x misaligned or I % 4 != 0: the register GEMV keeps its grouped range
    if (g_cfg.force_path == 0 && S <= group_gemv_limit(fmt)) {
        *gp = wq::plan_gemv(fmt, O, I, S, cus, g_cfg.waves_per_cu);
        if (gp->ok) return 1;
    }
    return 2;
}

// The workspace of stream `st`, grown to at least `bytes`. Only calls on
// `st` use it, and they run in stream order, so it is reused without any
// wait. Growing it, or handing a new stream the slot of the least recently
// used one (every slot taken), waits for the device to go idle (the old
// buffer may still be read). A call being captured into a graph never
// waits or allocates: it takes its stream's workspace if that is large
// enough, else the largest one that is (the graph then shares that
// stream's buffer), else it is refused.
int ensure_workspace(DeviceCtx &d, size_t bytes, hipStream_t st, uint16_t **out) {
    std::lock_guard<std::recursive_mutex> lk(d.mu);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return WQ_E_HIP;
    }
    DeviceCtx::StreamWs *e = nullptr;
    for (DeviceCtx::StreamWs &c : d.ws)
        if (c.live && c.st == st) e = &c;
    if (cs != hipStreamCaptureStatusNone) {
        if (e == nullptr || e->cap < bytes) {
            e = nullptr;
            for (DeviceCtx::StreamWs &c : d.ws)
                if (c.live && c.cap >= bytes && (e == nullptr || c.cap > e->cap)) e = &c;
        }
        if (e == nullptr) return WQ_E_UNSUPPORTED;
        *out = e->p;
        return WQ_OK;
    }
    const bool adopt = e == nullptr;
    if (adopt) {
        for (DeviceCtx::StreamWs &c : d.ws)
            if (!c.live && e == nullptr) e = &c;
        if (e == nullptr) {
            e = &d.ws[0];
            for (DeviceCtx::StreamWs &c : d.ws)
                if (c.last < e->last) e = &c;
        }
    }
    // a taken-over slot may still be read by its previous stream's calls
    if (bytes > e->cap || (adopt && e->live)) {
        if (hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            return WQ_E_HIP;
        }
    }
    if (bytes > e->cap) {
        dev_free(d, e->p, e->cap);
        e->p = nullptr;
        e->cap = 0;
        const size_t cap = (size_t)wq::round_up((long)bytes, 2L << 20);
        int rc = dev_alloc(d, (void **)&e->p, cap);
        if (rc != WQ_OK) {
            e->live = false;
            return rc;
        }
        e->cap = cap;
    }
    e->st = st;
    e->live = true;
    e->last = ++d.ws_clock;
    *out = e->p;
    return WQ_OK;
}

// fixed_ws != nullptr: the workspace is that buffer of fixed_cap bytes (the
// no-allocation entry point); a call needing more returns WQ_E_UNSUPPORTED
// before any launch. Otherwise the stream's workspace, grown on demand.
int run_matmul(const wq_tensor *t, const float *x, int S, float *y, hipStream_t st, uint16_t *fixed_ws = nullptr,
               size_t fixed_cap = 0) {
    DeviceCtx &d = g_dev[t->device];
    wq::GemvPlan gp;
    wq::SkinnyPlan skp;
    const bool x_vec = ((uintptr_t)x & 15) == 0;
    const int path = choose_path(t->fmt, t->O, t->I, S, d.cus, &gp, t->gs, x_vec, &skp);
    if (path == 3) {
        wq::SkinnyArgs a;
        a.w = t->d_w;
        a.scales = t->d_scales;
        a.x = x;
        a.y = y;
        a.stride = t->stride;
        a.nfull = t->nfull;
        a.O = t->O;
        a.I = t->I;
        a.S = S;
        a.chunks_per_wave = skp.chunks_per_wave;
        a.nchunks = skp.nchunks;
        a.gscales_t = t->d_scales_t;
        a.gs = t->gs;
        a.ng = t->ng;
        return hip_status(wq::launch_skinny(t->fmt, skp, a, st));
    }
    if (path == 1) {
        wq::GemvArgs a;
        a.w = t->d_w;
        a.scales = t->d_scales;
        a.x = x;
        a.y = y;
        a.stride = t->stride;
        a.nfull = t->nfull;
        a.gs = t->gs;
        a.ng = t->ng;
        a.O = t->O;
        a.I = t->I;
        a.S = S;
        a.k = gp.k;
        a.team = gp.team;
        a.teams_per_block = gp.teams_per_block;
        a.rows_per_team = gp.rows_per_team;
        return hip_status(wq::launch_gemv(gp, a, st));
    }
    const wq::TiledPlan tp = wq::plan_tiled(t->fmt, t->O, t->I, S, g_cfg.tiled_mode, g_cfg.tiled_shape, t->gs);
    wq::TiledArgs a;
    a.w = t->d_w;
    a.scales = t->gs > 0 ? t->d_scales_t : t->d_scales;
    a.x = x;
    a.y = y;
    a.stride = t->stride;
    a.nfull = t->nfull;
    a.gs = t->gs;
    a.ng = t->ng;
    a.O = t->O;
    a.I = t->I;
    a.S = S;
    a.tiles_s = tp.tiles_s;
    a.tiles_o = tp.tiles_o;
    a.xp = nullptr;
    a.plane = (long)tp.sp * tp.kp;
    a.kp = tp.kp;
    if (tp.ws_bytes > 0) {
        uint16_t *ws = fixed_ws;
        if (fixed_ws != nullptr) {
            if (tp.ws_bytes > fixed_cap) return WQ_E_UNSUPPORTED;
        } else {
            int rc = ensure_workspace(d, tp.ws_bytes, st, &ws);
            if (rc != WQ_OK) return rc;
        }
        a.xp = ws;
        if (tp.ksplit > 1) {
            a.ksplit = tp.ksplit;
            a.part = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + tp.part_off);
        }
    }
    return hip_status(wq::launch_tiled(t->fmt, tp, a, st));
}

int ensure_scratch(DeviceCtx &d, size_t xb, size_t yb) {
    if (xb > d.x_cap) {
        if (d.d_x) (void)hipFree(d.d_x);
        d.d_x = nullptr;
        d.x_cap = 0;
        if (hipMalloc((void **)&d.d_x, xb) != hipSuccess) {
            (void)hipGetLastError();
            return WQ_E_OOM;
        }
        d.x_cap = xb;
    }
    if (yb > d.y_cap) {
        if (d.d_y) (void)hipFree(d.d_y);
        d.d_y = nullptr;
        d.y_cap = 0;
        if (hipMalloc((void **)&d.d_y, yb) != hipSuccess) {
            (void)hipGetLastError();
            return WQ_E_OOM;
        }
        d.y_cap = yb;
    }
    auto pinned = [](size_t bytes, float **h, float **dh, size_t *cap) {
        if (bytes <= *cap) return WQ_OK;
        if (*h) (void)hipHostFree(*h);
        *h = *dh = nullptr;
        *cap = 0;
        if (hipHostMalloc((void **)h, bytes, hipHostMallocMapped) != hipSuccess) {
            (void)hipGetLastError();
            *h = nullptr;
            return WQ_E_OOM;
        }
        if (hipHostGetDevicePointer((void **)dh, *h, 0) != hipSuccess || *dh == nullptr) {
            (void)hipGetLastError();
            (void)hipHostFree(*h);
            *h = *dh = nullptr;
            return WQ_E_HIP;
        }
        *cap = bytes;
        return WQ_OK;
    };
    int rc = pinned(xb, &d.h_x, &d.dh_x, &d.hx_cap);
    if (rc == WQ_OK) rc = pinned(yb, &d.h_y, &d.dh_y, &d.hy_cap);
    return rc;
}

} // namespace

extern "C" {

int wq_init(const int *devices, int ndev) {
    if (ndev < 0 || ndev > WQ_MAX_DEVICES) return WQ_E_INVAL;
    if (ndev > 0 && devices == nullptr) return WQ_E_INVAL;
    int list[WQ_MAX_DEVICES];
    int n = ndev;
    if (ndev == 0) {
        list[0] = 0;
        n = 1;
    } else {
        for (int i = 0; i < ndev; ++i) {
            if (devices[i] < 0 || devices[i] >= WQ_MAX_DEVICES) return WQ_E_INVAL;
            for (int j = 0; j < i; ++j)
                if (devices[j] == devices[i]) return WQ_E_INVAL;
            list[i] = devices[i];
        }
    }
    std::lock_guard<std::mutex> lk(g_init_mu);
    read_env(g_cfg);
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return WQ_E_NODEV;
    }
    for (int i = 0; i < n; ++i)
        if (list[i] >= count) return WQ_E_INVAL;
    for (int i = 0; i < n; ++i) {
        DeviceCtx &d = g_dev[list[i]];
        if (d.open) continue;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, list[i]) != hipSuccess) return WQ_E_HIP;
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return WQ_E_NODEV;
        DeviceGuard guard(list[i]);
        // hipGetSymbolAddress acts on the current device: the guard made
        // list[i] current (each device holds its own copy of `scratch`)
        void *sp = nullptr;
        if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || sp == nullptr) {
            (void)hipGetLastError();
            return WQ_E_HIP;
        }
        hipStream_t st = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return WQ_E_HIP;
        d.scratch = static_cast<uint16_t *>(sp);
        d.stream = st;
        d.cus = prop.multiProcessorCount;
        d.total_mem = prop.totalGlobalMem;
        snprintf(d.name, sizeof d.name, "%s", prop.name);
        snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
        d.open = true;
        if (g_cfg.verbose)
            fprintf(stderr, "wqmm: device %d: %s (%s), %.1f GiB, %d CUs\n", list[i], d.name, d.arch,
                    d.total_mem / 1073741824.0, d.cus);
    }
    return WQ_OK;
}

int wq_mem_info(int device, size_t *free_b, size_t *total_b) {
    if (device < 0 || device >= WQ_MAX_DEVICES) return WQ_E_INVAL;
    if (!device_open(device)) return WQ_E_NOTINIT;
    DeviceGuard guard(device);
    size_t f = 0, t = 0;
    if (hipMemGetInfo(&f, &t) != hipSuccess) return WQ_E_HIP;
    if (free_b) *free_b = f;
    if (total_b) *total_b = t;
    return WQ_OK;
}

long wq_row_bytes(int fmt, long I) { return wq::row_bytes(fmt, I); }

} // extern "C"

namespace {

// gs == 0: one scale per row (device rows permuted in 1 KiB blocks);
// gs > 0: O x ceil(I/gs) scales, rows kept in natural element order.
int upload_impl(wq_tensor **t, int device, int fmt, int O, int I, int gs, const void *w, const float *scales) {
    if (t == nullptr) return WQ_E_INVAL;
    if (!valid_fmt(fmt) || O <= 0 || I <= 0 || device < 0 || device >= WQ_MAX_DEVICES || gs < 0)
        return WQ_E_INVAL;
    if (gs > 0 && fmt == WQ_F32) return WQ_E_INVAL;  // scales apply to quantized weights only
    if (gs > 0 && gs % wq::kGroupAlign != 0) return WQ_E_UNSUPPORTED;
    if (*t != nullptr) {
        const wq_tensor *r = *t;
        if (!tensor_ok(r)) return WQ_E_INVAL;
        if (r->device != device || r->fmt != fmt || r->O != O || r->I != I || r->gs != gs) return WQ_E_MISMATCH;
        return WQ_OK;
    }
    if (w == nullptr) return WQ_E_INVAL;
    if (scales == nullptr && fmt != WQ_F32) return WQ_E_INVAL;
    if (!device_open(device)) return WQ_E_NOTINIT;
    if (g_cfg.fault == 1) return WQ_E_FAULT;
    DeviceCtx &d = g_dev[device];
    std::lock_guard<std::recursive_mutex> lk(d.mu);
    DeviceGuard guard(device);

    const long rb = wq::row_bytes(fmt, I);
    const long stride = wq::round_up(rb, wq::kRowAlign);
    const int ng = gs > 0 ? (int)(((long)I + gs - 1) / gs) : 1;
    const size_t wbytes = (size_t)O * stride;
    const size_t sbytes = (size_t)O * ng * sizeof(float);
    void *dw = nullptr, *ds = nullptr, *dst_t = nullptr;
    int rc = dev_alloc(d, &dw, wbytes);
    if (rc != WQ_OK) return rc;
    rc = dev_alloc(d, &ds, sbytes);
    if (rc == WQ_OK && gs > 0) rc = dev_alloc(d, &dst_t, sbytes);
    if (rc != WQ_OK) {
        dev_free(d, dw, wbytes);
        dev_free(d, ds, sbytes);
        return rc;
    }
    auto free_all = [&]() {
        dev_free(d, dw, wbytes);
        dev_free(d, ds, sbytes);
        if (dst_t) dev_free(d, dst_t, sbytes);
    };
    const int nfull = gs > 0 ? 0 : wq::full_blocks(fmt, rb);
    hipError_t e = hipSuccess;
    if (nfull == 0) {
        // natural order: copy rows into the padded stride
        if (stride != rb) {
            e = hipMemsetAsync(dw, 0, wbytes, d.stream);
            if (e == hipSuccess)
                e = hipMemcpy2DAsync(dw, stride, w, rb, rb, O, hipMemcpyHostToDevice, d.stream);
        } else {
            e = hipMemcpyAsync(dw, w, wbytes, hipMemcpyHostToDevice, d.stream);
        }
    } else {
        // stage the natural rows, then permute 1 KiB blocks into the device layout
        void *tmp = nullptr;
        if (hipMalloc(&tmp, (size_t)O * rb) != hipSuccess) {
            (void)hipGetLastError();
            free_all();
            return WQ_E_OOM;
        }
        e = hipMemcpyAsync(tmp, w, (size_t)O * rb, hipMemcpyHostToDevice, d.stream);
        if (e == hipSuccess)
            e = wq::launch_relayout(fmt, (const uint8_t *)tmp, (uint8_t *)dw, O, rb, stride, nfull, d.stream);
        hipError_t e2 = hipStreamSynchronize(d.stream);
        if (e == hipSuccess) e = e2;
        (void)hipFree(tmp);
    }
    std::vector<float> ones;
    if (e == hipSuccess) {
        const float *src = scales;
        if (src == nullptr) {  // f32 without scales (gs == 0 only)
            ones.assign(O, 1.0f);
            src = ones.data();
        }
        e = hipMemcpyAsync(ds, src, sbytes, hipMemcpyHostToDevice, d.stream);
    }
    std::vector<float> st;
    if (e == hipSuccess && gs > 0) {  // group-major copy for the tiled path
        st.resize((size_t)O * ng);
        for (long o = 0; o < O; ++o)
            for (long g = 0; g < ng; ++g) st[(size_t)g * O + o] = scales[(size_t)o * ng + g];
        e = hipMemcpyAsync(dst_t, st.data(), sbytes, hipMemcpyHostToDevice, d.stream);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(d.stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        free_all();
        return hip_status(e);
    }
    wq_tensor *nt = new (std::nothrow) wq_tensor;
    if (!nt) {
        free_all();
        return WQ_E_OOM;
    }
    nt->magic = wq::kTensorMagic;
    nt->device = device;
    nt->fmt = fmt;
    nt->O = O;
    nt->I = I;
    nt->rb = rb;
    nt->stride = stride;
    nt->nfull = nfull;
    nt->gs = gs;
    nt->ng = ng;
    nt->d_w = (uint8_t *)dw;
    nt->d_scales = (float *)ds;
    nt->d_scales_t = (float *)dst_t;
    nt->bytes = wbytes + sbytes * (gs > 0 ? 2 : 1);
    *t = nt;
    return WQ_OK;
}

} // namespace

extern "C" {

int wq_tensor_upload(wq_tensor **t, int device, int fmt, int O, int I, const void *w, const float *scales) {
    return upload_impl(t, device, fmt, O, I, 0, w, scales);
}

int wq_tensor_upload_gs(wq_tensor **t, int device, int fmt, int O, int I, int gs, const void *w,
                        const float *scales) {
    if (gs <= 0) return WQ_E_INVAL;
    return upload_impl(t, device, fmt, O, I, gs, w, scales);
}

int wq_matmul_t(const wq_tensor *t, const float *x, int S, float *y) {
    if (!tensor_ok(t) || S < 0) return WQ_E_INVAL;
    if (S == 0) return WQ_OK;
    if (x == nullptr || y == nullptr) return WQ_E_INVAL;
    if (!device_open(t->device)) return WQ_E_NOTINIT;
    if (g_cfg.fault == 2) return WQ_E_FAULT;
    DeviceCtx &d = g_dev[t->device];
    std::lock_guard<std::recursive_mutex> lk(d.mu);
    DeviceGuard guard(t->device);
    const size_t xb = (size_t)S * t->I * sizeof(float);
    const size_t yb = (size_t)S * t->O * sizeof(float);
    int rc = ensure_scratch(d, xb, yb);
    if (rc != WQ_OK) return rc;
    // x -> pinned staging -> device by a copy kernel, the matmul, y back the
    // same way; the previous call finished before it returned, so the
    // staging buffers are free
    memcpy(d.h_x, x, xb);
    hipError_t e = wq::launch_stage_copy(d.dh_x, d.d_x, xb / sizeof(float), d.stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_status(e);
    }
    rc = run_matmul(t, d.d_x, S, d.d_y, d.stream);
    if (rc != WQ_OK) {
        (void)hipStreamSynchronize(d.stream);
        return rc;
    }
    e = wq::launch_stage_copy(d.d_y, d.dh_y, yb / sizeof(float), d.stream);
    if (e == hipSuccess) e = hipStreamSynchronize(d.stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_status(e);
    }
    memcpy(y, d.h_y, yb);  // y is written only on success
    return WQ_OK;
}

int wq_matmul(wq_tensor **t, int device, int fmt, int O, int I, const void *w, const float *scales,
              const float *x, int S, float *y) {
    if (S < 0) return WQ_E_INVAL;
    if (S > 0 && (x == nullptr || y == nullptr)) return WQ_E_INVAL;
    int rc = wq_tensor_upload(t, device, fmt, O, I, w, scales);
    if (rc != WQ_OK) return rc;
    return wq_matmul_t(*t, x, S, y);
}

int wq_matmul_dev(const wq_tensor *t, const float *x_dev, int S, float *y_dev, void *hip_stream) {
    if (!tensor_ok(t) || S < 0) return WQ_E_INVAL;
    if (S == 0) return WQ_OK;
    if (x_dev == nullptr || y_dev == nullptr) return WQ_E_INVAL;
    if (((uintptr_t)x_dev & 3) || ((uintptr_t)y_dev & 3)) return WQ_E_INVAL;
    if (!device_open(t->device)) return WQ_E_NOTINIT;
    if (g_cfg.fault == 2) return WQ_E_FAULT;
    DeviceGuard guard(t->device);
    return run_matmul(t, x_dev, S, y_dev, (hipStream_t)hip_stream);
}

int wq_matmul_dev_noalloc(const wq_tensor *t, const float *x_dev, int S, float *y_dev, void *hip_stream) {
    if (!tensor_ok(t) || S < 0) return WQ_E_INVAL;
    if (S == 0) return WQ_OK;
    if (x_dev == nullptr || y_dev == nullptr) return WQ_E_INVAL;
    if (((uintptr_t)x_dev & 3) || ((uintptr_t)y_dev & 3)) return WQ_E_INVAL;
    if (!device_open(t->device)) return WQ_E_NOTINIT;
    if (g_cfg.fault == 2) return WQ_E_FAULT;
    DeviceCtx &d = g_dev[t->device];
    if (d.scratch == nullptr) return WQ_E_NOTINIT;
    DeviceGuard guard(t->device);
    return run_matmul(t, x_dev, S, y_dev, (hipStream_t)hip_stream, d.scratch, kScratchBytes);
}

size_t wq_noalloc_scratch_bytes(void) { return kScratchBytes; }

} // extern "C"

namespace {

// A group of G problems; ts2 != nullptr makes it a paired group (problem i is
// gate ts[i] with up ts2[i], same shape), whose work items count virtual rows.
int create_group(wq_tensor *const *ts, wq_tensor *const *ts2, int G, wq_group **group) {
    if (ts == nullptr || group == nullptr || G <= 0) return WQ_E_INVAL;
    for (int i = 0; i < G; ++i)
        if (!tensor_ok(ts[i]) || (ts2 && !tensor_ok(ts2[i]))) return WQ_E_INVAL;
    const int dev = ts[0]->device, fmt = ts[0]->fmt;
    for (int i = 1; i < G; ++i)
        if (ts[i]->device != dev || ts[i]->fmt != fmt) return WQ_E_INVAL;
    if (ts2) {
        for (int i = 0; i < G; ++i) {
            const wq_tensor *a = ts[i], *b = ts2[i];
            if (b->device != dev || b->fmt != fmt || b->O != a->O || b->I != a->I || b->gs != a->gs ||
                b->stride != a->stride || b->nfull != a->nfull)
                return WQ_E_INVAL;
        }
    }
    if (!device_open(dev)) return WQ_E_NOTINIT;
    DeviceCtx &d = g_dev[dev];
    std::lock_guard<std::recursive_mutex> lk(d.mu);
    DeviceGuard guard(dev);

    wq_group *g = new (std::nothrow) wq_group;
    if (!g) return WQ_E_OOM;
    g->magic = wq::kGroupMagic;
    g->device = dev;
    g->fmt = fmt;
    g->G = G;
    g->ts.assign(ts, ts + G);
    if (ts2) g->ts2.assign(ts2, ts2 + G);
    g->d_desc = nullptr;
    const int vrows = ts2 ? 2 : 1;  // virtual rows per output row
    for (int i = 0; i < G; ++i) {
        wq::GroupDesc gd;
        gd.w = ts[i]->d_w;
        gd.scales = ts[i]->d_scales;
        gd.w2 = ts2 ? ts2[i]->d_w : nullptr;
        gd.scales2 = ts2 ? ts2[i]->d_scales : nullptr;
        gd.stride = ts[i]->stride;
        gd.nfull = ts[i]->nfull;
        gd.O = ts[i]->O;
        gd.I = ts[i]->I;
        gd.pad = 0;
        g->h_desc.push_back(gd);
        if (ts[i]->gs > 0 || (ts2 && ts2[i]->gs > 0)) g->has_gs = true;
    }
    auto fail = [&](int rc) {
        for (auto &b : g->buckets)
            if (b.d_items) dev_free(d, b.d_items, (size_t)b.plan.n_items * sizeof(wq::WorkItem));
        if (g->d_desc) dev_free(d, g->d_desc, (size_t)G * sizeof(wq::GroupDesc));
        g->magic = 0;
        delete g;
        return rc;
    };
    int rc = dev_alloc(d, (void **)&g->d_desc, (size_t)G * sizeof(wq::GroupDesc));
    if (rc != WQ_OK) return fail(rc);
    hipError_t e = hipMemcpyAsync(g->d_desc, g->h_desc.data(), (size_t)G * sizeof(wq::GroupDesc),
                                  hipMemcpyHostToDevice, d.stream);
    if (e != hipSuccess) return fail(hip_status(e));
    // Work tables for every S bucket, built now so later calls never allocate.
    for (int bi = 0; bi < 4; ++bi) {
        auto &bk = g->buckets[bi];
        const int smax = 1 << bi;
        const wq::GemvShape sh = wq::gemv_shape(fmt, smax);
        bk = wq_group::Bucket();
        bk.plan.smax = smax;
        bk.plan.lw = sh.lw;
        bk.plan.kmax = sh.kmax;
        bk.plan.d = sh.d;
        const long per_wave = 64L * sh.lw * sh.kmax;
        bool fits = true;
        for (const auto &gd : g->h_desc)
            if (gd.stride > per_wave) fits = false;
        if (!fits) continue;
        // One launch per chunk of <= kGroupMaxPerLaunch problems, whatever
        // their row lengths: the chunk's weight bytes are cut into about
        // cus * waves_per_cu items of equal bytes, each a row range of one
        // problem (a multiple of the ring depth its slot count runs with).
        // A chunk whose rows all need the same slot count runs the kernel
        // compiled for exactly that count (8 waves per CU); otherwise the
        // kernel that picks the count per item, whose registers (those of
        // the longest rows, about 150 at S = 1) allow 3 waves per SIMD: 12
        // items per CU fill exactly one resident round (measured on the
        // 8-expert int4 layer, 24 matmuls: 31.4 us at 12 per CU, 37.2 at 10,
        // 36.3 at 14, where part of the work waits for a second round).
        auto slots = [&](const wq::GroupDesc &gd) { return (int)((gd.stride + 64L * sh.lw - 1) / (64L * sh.lw)); };
        std::vector<wq::WorkItem> items;
        for (int c0 = 0; c0 < G; c0 += wq::kGroupMaxPerLaunch) {
            const int c1 = std::min(G, c0 + wq::kGroupMaxPerLaunch);
            long seg_bytes = 0;
            uint64_t mask = 0;
            int k_first = 0;
            bool one_k = true;
            for (int p = c0; p < c1; ++p) {
                seg_bytes += (long)vrows * g->h_desc[p].O * g->h_desc[p].stride;
                mask |= 1ull << (p - c0);
                const int k = slots(g->h_desc[p]);
                if (p == c0) k_first = k;
                one_k = one_k && k == k_first;
            }
            const int wpc = g_cfg.waves_per_cu > 0 ? g_cfg.waves_per_cu : one_k ? 8 : 12;
            const long target_items = std::max(1L, (long)d.cus * wpc);
            const long bytes_per_item = std::max(1L, (seg_bytes + target_items - 1) / target_items);
            const int first = (int)items.size();
            for (int p = c0; p < c1; ++p) {
                const auto &gd = g->h_desc[p];
                const int k = slots(gd);
                const int dk = wq::ring_depth(sh.kmax, sh.d, k);  // the kernel's ring depth for k slots
                long rows = (bytes_per_item + gd.stride - 1) / gd.stride;
                rows = std::max<long>(dk, (rows + dk - 1) / dk * dk);
                const long nrows = (long)vrows * gd.O;
                for (long r0 = 0; r0 < nrows; r0 += rows) {
                    wq::WorkItem it;
                    it.p = p - c0;
                    it.row_begin = (int)r0;
                    it.row_end = (int)std::min<long>(nrows, r0 + rows);
                    it.k = k;
                    items.push_back(it);
                }
            }
            bk.seg_chunk.push_back(c0 / wq::kGroupMaxPerLaunch);
            bk.first_item.push_back(first);
            bk.n_items.push_back((int)items.size() - first);
            bk.ks.push_back(one_k ? k_first : 0);
            bk.mask.push_back(mask);
        }
        bk.plan.n_items = (int)items.size();
        rc = dev_alloc(d, (void **)&bk.d_items, items.size() * sizeof(wq::WorkItem));
        if (rc != WQ_OK) return fail(rc);
        e = hipMemcpyAsync(bk.d_items, items.data(), items.size() * sizeof(wq::WorkItem),
                           hipMemcpyHostToDevice, d.stream);
        if (e != hipSuccess) return fail(hip_status(e));
        e = hipStreamSynchronize(d.stream);  // `items` goes out of scope
        if (e != hipSuccess) return fail(hip_status(e));
        bk.plan.ok = true;
        bk.built = true;
    }
    e = hipStreamSynchronize(d.stream);
    if (e != hipSuccess) return fail(hip_status(e));
    *group = g;
    return WQ_OK;
}

// One expert's gated front half: h[S, O] = silu(gate . x) * (up . x).
// S within the grouped GEMV limit and one scale per row: one paired-row
// launch (both dot products of an output from one read of x). Otherwise
// gate -> h and up -> u (in the stream's workspace, after the tiled planes
// when the matmuls take the tiled path) as two ordinary matmuls, then the
// in-place activation kernel.
int run_swiglu(const wq_tensor *gt, const wq_tensor *ut, const float *x, int S, float *h, hipStream_t st) {
    DeviceCtx &d = g_dev[gt->device];
    wq::GemvPlan gp;
    bool paired = false;
    if (gt->gs == 0 && g_cfg.force_path != 2 && g_cfg.force_path != 3 && S <= group_gemv_limit(gt->fmt)) {
        gp = wq::plan_gemv(gt->fmt, 2 * gt->O, gt->I, S, d.cus, g_cfg.waves_per_cu);
        paired = gp.ok;
    }
    if (paired) {
        wq::GemvArgs a;
        a.w = gt->d_w;
        a.scales = gt->d_scales;
        a.w2 = ut->d_w;
        a.scales2 = ut->d_scales;
        a.x = x;
        a.y = h;
        a.stride = gt->stride;
        a.nfull = gt->nfull;
        a.gs = 0;
        a.ng = 1;
        a.O = 2 * gt->O;
        a.I = gt->I;
        a.S = S;
        a.k = gp.k;
        a.team = gp.team;
        a.teams_per_block = gp.teams_per_block;
        a.rows_per_team = gp.rows_per_team;
        return hip_status(wq::launch_gemv(gp, a, st));
    }
    size_t planes = 0;  // the path run_matmul will take for gate and up (same shape and x)
    if (choose_path(gt->fmt, gt->O, gt->I, S, d.cus, &gp, gt->gs, ((uintptr_t)x & 15) == 0) == 2)
        planes = wq::plan_tiled(gt->fmt, gt->O, gt->I, S, g_cfg.tiled_mode, g_cfg.tiled_shape, gt->gs).ws_bytes;
    const size_t off = (size_t)wq::round_up((long)planes, 256);
    uint16_t *ws = nullptr;
    int rc = ensure_workspace(d, off + (size_t)S * gt->O * sizeof(float), st, &ws);
    if (rc != WQ_OK) return rc;
    float *u = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + off);
    rc = run_matmul(gt, x, S, h, st);
    if (rc == WQ_OK) rc = run_matmul(ut, x, S, u, st);
    if (rc == WQ_OK) rc = hip_status(wq::launch_gated_inplace(h, u, (long)S * gt->O, st));
    return rc;
}

// The group-scale fields of a grouped few-rows descriptor: a tensor with one
// scale per row is one group as long as the row.
void set_group_scales(wq::SkinnyGroupDesc &e, const wq_tensor *t) {
    e.gscales_t = t->gs > 0 ? t->d_scales_t : t->d_scales;
    e.gs = t->gs > 0 ? t->gs : (1 << 30);
    e.ng = t->gs > 0 ? t->ng : 1;
}

// Shared by the plain and the paired group calls (checked by the callers).
int run_group(wq_group *g, const float *const *x_dev, const int *S, float *const *y_dev, hipStream_t st) {
    const bool pair = !g->ts2.empty();
    int smax = 0;
    for (int i = 0; i < g->G; ++i) {
        if (S[i] < 0) return WQ_E_INVAL;
        if (S[i] > 0) {
            if (x_dev[i] == nullptr || y_dev[i] == nullptr) return WQ_E_INVAL;
            if (((uintptr_t)x_dev[i] & 3) || ((uintptr_t)y_dev[i] & 3)) return WQ_E_INVAL;
            if (!tensor_ok(g->ts[i]) || (pair && !tensor_ok(g->ts2[i]))) return WQ_E_INVAL;
        }
        smax = std::max(smax, S[i]);
    }
    if (smax == 0) return WQ_OK;
    if (!device_open(g->device)) return WQ_E_NOTINIT;
    if (g_cfg.fault == 2) return WQ_E_FAULT;
    DeviceGuard guard(g->device);
    const int bucket = wq::gemv_smax_bucket(smax);
    const int bi = bucket == 1 ? 0 : bucket == 2 ? 1 : bucket == 4 ? 2 : bucket == 8 ? 3 : -1;
    const bool one_launch = !g->has_gs && g_cfg.force_path != 2 && g_cfg.force_path != 3 &&
                            smax <= group_gemv_limit(g->fmt) && bi >= 0 && g->buckets[bi].plan.ok;
    if (!one_launch && !pair && g_cfg.force_path == 0) {
        // up to 32 rows per tensor (16 with group scales): the few-rows
        // kernel over the whole group, one launch per kSkinnyGroupMax active
        // tensors
        wq::SkinnyGroupArgs a;
        memset(&a, 0, sizeof a);
        std::vector<wq::SkinnyGroupArgs> launches;
        std::vector<wq::SkinnyGroupPlan> plans;
        bool ok = true;
        for (int i = 0; i < g->G && ok; ++i) {
            if (S[i] == 0) continue;
            const wq_tensor *t = g->ts[i];
            if (((uintptr_t)x_dev[i] & 15) != 0 || t->stride >= INT_MAX) ok = false;
            wq::SkinnyGroupDesc &e = a.t[a.n++];
            e.w = t->d_w;
            e.scales = t->d_scales;
            e.x = x_dev[i];
            e.y = y_dev[i];
            e.stride = (int)t->stride;
            e.nfull = t->nfull;
            e.O = t->O;
            e.I = t->I;
            e.S = S[i];
            set_group_scales(e, t);
            if (a.n == wq::kSkinnyGroupMax) {
                launches.push_back(a);
                memset(&a, 0, sizeof a);
            }
        }
        if (a.n > 0) launches.push_back(a);
        for (size_t c = 0; c < launches.size() && ok; ++c) {
            plans.push_back(
                wq::plan_skinny_group(g->fmt, launches[c].t, launches[c].n, g_dev[g->device].cus, g->has_gs));
            ok = plans.back().ok;
        }
        if (ok) {
            for (size_t c = 0; c < launches.size(); ++c) {
                int rc = hip_status(wq::launch_skinny_group(g->fmt, plans[c], launches[c], st));
                if (rc != WQ_OK) return rc;
            }
            return WQ_OK;
        }
    }
    if (!one_launch && pair && g_cfg.force_path == 0) {
        // up to 32 rows per expert, gated: gate -> h and up -> u (in the
        // stream's workspace) of every expert in grouped few-rows launches,
        // then one activation launch per kSkinnyGroupMax experts
        std::vector<int> act;
        bool ok = true;
        size_t ubytes = 0;
        std::vector<size_t> uoff(g->G, 0);
        for (int i = 0; i < g->G; ++i) {
            if (S[i] == 0) continue;
            if (((uintptr_t)x_dev[i] & 15) != 0 || g->ts[i]->stride >= INT_MAX || S[i] > wq::kSkinnyMaxS) ok = false;
            act.push_back(i);
            uoff[i] = ubytes;
            ubytes += (size_t)wq::round_up((long)S[i] * g->ts[i]->O * (long)sizeof(float), 256);
        }
        std::vector<wq::SkinnyGroupArgs> launches;
        std::vector<wq::SkinnyGroupPlan> plans;
        const int per = wq::kSkinnyGroupMax / 2;  // experts per launch (two tensors each)
        for (size_t c = 0; c < act.size() && ok; c += per) {
            wq::SkinnyGroupArgs a;
            memset(&a, 0, sizeof a);
            for (size_t j = c; j < std::min(act.size(), c + per); ++j) {
                const int i = act[j];
                for (int h = 0; h < 2; ++h) {
                    const wq_tensor *t = h ? g->ts2[i] : g->ts[i];
                    wq::SkinnyGroupDesc &e = a.t[a.n++];
                    e.w = t->d_w;
                    e.scales = t->d_scales;
                    e.x = x_dev[i];
                    e.y = y_dev[i];  // up: set once the workspace is known
                    e.stride = (int)t->stride;
                    e.nfull = t->nfull;
                    e.O = t->O;
                    e.I = t->I;
                    e.S = S[i];
                    set_group_scales(e, t);
                }
            }
            plans.push_back(wq::plan_skinny_group(g->fmt, a.t, a.n, g_dev[g->device].cus, g->has_gs));
            ok = plans.back().ok;
            launches.push_back(a);
        }
        if (ok && !act.empty()) {
            uint16_t *ws = nullptr;
            int rc = ensure_workspace(g_dev[g->device], ubytes, st, &ws);
            if (rc != WQ_OK) return rc;
            char *ub = reinterpret_cast<char *>(ws);
            for (size_t c = 0; c < launches.size(); ++c) {
                for (int k = 1; k < launches[c].n; k += 2)
                    launches[c].t[k].y = reinterpret_cast<float *>(ub + uoff[act[c * per + k / 2]]);
                rc = hip_status(wq::launch_skinny_group(g->fmt, plans[c], launches[c], st));
                if (rc != WQ_OK) return rc;
            }
            for (size_t c = 0; c < act.size(); c += wq::kSkinnyGroupMax) {
                wq::GatedGroupArgs ga;
                memset(&ga, 0, sizeof ga);
                int maxc = 0;
                for (size_t j = c; j < std::min(act.size(), c + wq::kSkinnyGroupMax); ++j) {
                    const int i = act[j];
                    auto &e = ga.e[ga.n++];
                    e.h = y_dev[i];
                    e.u = reinterpret_cast<const float *>(ub + uoff[i]);
                    e.count = S[i] * g->ts[i]->O;
                    maxc = std::max(maxc, e.count);
                }
                rc = hip_status(wq::launch_gated_group(ga, maxc, st));
                if (rc != WQ_OK) return rc;
            }
            return WQ_OK;
        }
    }
    if (!one_launch) {
        for (int i = 0; i < g->G; ++i) {
            if (S[i] == 0) continue;
            int rc = pair ? run_swiglu(g->ts[i], g->ts2[i], x_dev[i], S[i], y_dev[i], st)
                          : run_matmul(g->ts[i], x_dev[i], S[i], y_dev[i], st);
            if (rc != WQ_OK) return rc;
        }
        return WQ_OK;
    }
    const auto &bk = g->buckets[bi];
    for (size_t c = 0; c < bk.first_item.size(); ++c) {  // one launch per segment
        const int c0 = bk.seg_chunk[c] * wq::kGroupMaxPerLaunch;
        const int c1 = std::min(g->G, c0 + wq::kGroupMaxPerLaunch);
        bool any = false;
        wq::GroupedArgs a;
        memset(&a, 0, sizeof a);
        a.desc = g->d_desc + c0;
        a.items = bk.d_items + bk.first_item[c];
        a.n_items = bk.n_items[c];
        for (int p = c0; p < c1; ++p) {
            a.x[p - c0] = x_dev[p];
            a.y[p - c0] = y_dev[p];
            a.S[p - c0] = S[p];
            if ((bk.mask[c] >> (p - c0)) & 1) any = any || S[p] > 0;
        }
        if (!any || a.n_items == 0) continue;
        bool xv = true;
        for (int p = c0; p < c1; ++p)
            if (S[p] > 0 && ((g->h_desc[p].I % 4) != 0 || ((uintptr_t)x_dev[p] & 15) != 0)) xv = false;
        wq::GroupedPlan gp = bk.plan;
        gp.grid = (a.n_items + 3) / 4;
        gp.block = 256;
        int rc = hip_status(wq::launch_grouped(g->fmt, gp, a, xv, pair, bk.ks[c], st));
        if (rc != WQ_OK) return rc;
    }
    return WQ_OK;
}

} // namespace

extern "C" {

int wq_grouped_create(wq_tensor *const *ts, int G, wq_group **group) {
    return create_group(ts, nullptr, G, group);
}

int wq_swiglu_create(wq_tensor *const *gate, wq_tensor *const *up, int E, wq_group **group) {
    if (up == nullptr) return WQ_E_INVAL;
    return create_group(gate, up, E, group);
}

int wq_swiglu_matmul_dev(wq_group *g, const float *const *x_dev, const int *S, float *const *h_dev,
                         void *hip_stream) {
    if (g == nullptr || g->magic != wq::kGroupMagic || g->ts2.empty()) return WQ_E_INVAL;
    if (x_dev == nullptr || S == nullptr || h_dev == nullptr) return WQ_E_INVAL;
    return run_group(g, x_dev, S, h_dev, (hipStream_t)hip_stream);
}

int wq_swiglu_ffn_dev(wq_group *gu, wq_group *down, const float *const *x_dev, const int *S,
                      float *const *h_dev, float *const *y_dev, void *hip_stream) {
    if (gu == nullptr || gu->magic != wq::kGroupMagic || gu->ts2.empty()) return WQ_E_INVAL;
    if (down == nullptr || down->magic != wq::kGroupMagic || !down->ts2.empty()) return WQ_E_INVAL;
    if (x_dev == nullptr || S == nullptr || h_dev == nullptr || y_dev == nullptr) return WQ_E_INVAL;
    if (down->G != gu->G || down->device != gu->device) return WQ_E_INVAL;
    for (int e = 0; e < gu->G; ++e)
        if (!tensor_ok(down->ts[e]) || !tensor_ok(gu->ts[e]) || down->ts[e]->I != gu->ts[e]->O)
            return WQ_E_INVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    int rc = run_group(gu, x_dev, S, h_dev, st);
    if (rc != WQ_OK) return rc;
    return run_group(down, h_dev, S, y_dev, st);
}

int wq_grouped_matmul_dev(wq_group *g, const float *const *x_dev, const int *S, float *const *y_dev,
                          void *hip_stream) {
    if (g == nullptr || g->magic != wq::kGroupMagic || !g->ts2.empty()) return WQ_E_INVAL;
    if (x_dev == nullptr || S == nullptr || y_dev == nullptr) return WQ_E_INVAL;
    return run_group(g, x_dev, S, y_dev, (hipStream_t)hip_stream);
}

int wq_grouped_free(wq_group *g) {
    if (g == nullptr) return WQ_OK;
    if (g->magic != wq::kGroupMagic) return WQ_E_INVAL;
    DeviceCtx &d = g_dev[g->device];
    std::lock_guard<std::recursive_mutex> lk(d.mu);
    DeviceGuard guard(g->device);
    for (auto &b : g->buckets)
        if (b.d_items) dev_free(d, b.d_items, (size_t)b.plan.n_items * sizeof(wq::WorkItem));
    if (g->d_desc) dev_free(d, g->d_desc, (size_t)g->G * sizeof(wq::GroupDesc));
    g->magic = 0;
    delete g;
    return WQ_OK;
}

int wq_tensor_free(wq_tensor *t) {
    if (t == nullptr) return WQ_OK;
    if (!tensor_ok(t)) return WQ_E_INVAL;
    DeviceCtx &d = g_dev[t->device];
    std::lock_guard<std::recursive_mutex> lk(d.mu);
    DeviceGuard guard(t->device);
    dev_free(d, t->d_w, (size_t)t->O * t->stride);
    dev_free(d, t->d_scales, (size_t)t->O * t->ng * sizeof(float));
    if (t->d_scales_t) dev_free(d, t->d_scales_t, (size_t)t->O * t->ng * sizeof(float));
    t->magic = 0;
    delete t;
    return WQ_OK;
}

const char *wq_strerror(int code) {
    switch (code) {
    case WQ_OK: return "success";
    case WQ_E_INVAL: return "invalid argument";
    case WQ_E_NODEV: return "no usable gfx950 device";
    case WQ_E_NOTINIT: return "device not initialised (call wq_init)";
    case WQ_E_OOM: return "out of device memory (or over WQ_MEM_LIMIT_BYTES)";
    case WQ_E_MISMATCH: return "resident tensor differs from the re-upload request";
    case WQ_E_HIP: return "HIP runtime error";
    case WQ_E_FAULT: return "injected failure (WQ_FAULT)";
    case WQ_E_UNSUPPORTED: return "unsupported request";
    default: return "unknown status code";
    }
}

int wq_stream_read_dev(const void *buf_dev, size_t bytes, int waves, int loads_in_flight, unsigned *out_dev,
                       void *hip_stream) {
    if (buf_dev == nullptr || out_dev == nullptr || waves <= 0 || waves % 4 != 0 || waves > (1 << 20)) return WQ_E_INVAL;
    if (((uintptr_t)buf_dev & 15) || ((uintptr_t)out_dev & 3) || bytes % 16 != 0) return WQ_E_INVAL;
    const int ok[] = {1, 2, 4, 5, 8, 9, 12, 16, 18, 24, 36};
    if (std::find(std::begin(ok), std::end(ok), loads_in_flight) == std::end(ok)) return WQ_E_INVAL;
    if (bytes == 0) return WQ_OK;
    return hip_status(wq::launch_stream_read(buf_dev, bytes, waves, loads_in_flight, out_dev, (hipStream_t)hip_stream));
}

int wq_describe_plan(int fmt, int O, int I, int S, char *buf, size_t buflen) {
    return wq_describe_plan_gs(fmt, O, I, S, 0, buf, buflen);
}

int wq_describe_plan_gs(int fmt, int O, int I, int S, int gs, char *buf, size_t buflen) {
    if (!valid_fmt(fmt) || O <= 0 || I <= 0 || S < 0 || gs < 0 || buf == nullptr || buflen == 0) return WQ_E_INVAL;
    const int cus = device_open(0) ? g_dev[0].cus : kDefaultCUs;
    if (S == 0) {
        snprintf(buf, buflen, "none");
        return WQ_OK;
    }
    wq::GemvPlan gp;
    wq::SkinnyPlan sp;
    const int path = choose_path(fmt, O, I, S, cus, &gp, gs, true, &sp);
    if (path == 1) {
        snprintf(buf, buflen, "gemv fmt=%d smax=%d lw=%d kmax=%d k=%d team=%d d=%d rows_per_team=%d grid=%d block=%d",
                 fmt, gp.smax, gp.lw, gp.kmax, gp.k, gp.team, gp.d, gp.rows_per_team, gp.grid, gp.block);
    } else if (path == 3) {
        snprintf(buf, buflen,
                 "skinny fmt=%d m=%d rpl=%d nb=%d waves=%d ring=%d chunks=%d chunks_per_wave=%d grid=%d block=%d "
                 "workspace=0",
                 fmt, sp.m, sp.rpl, sp.nb, sp.waves, sp.ring, sp.nchunks, sp.chunks_per_wave, sp.grid, 64 * sp.waves);
    } else {
        const wq::TiledPlan tp = wq::plan_tiled(fmt, O, I, S, g_cfg.tiled_mode, g_cfg.tiled_shape, gs);
        snprintf(buf, buflen,
                 "tiled fmt=%d mode=%s bm=%d bn=%d bk=%d tiles_s=%d tiles_o=%d ksplit=%d grid=%d block=%d "
                 "workspace=%zu",
                 fmt, tp.mode == wq::kTiledBF16X3 ? "bf16x3" : tp.mode == wq::kTiledBF16 ? "bf16" : "fp32", tp.bm, tp.bn, tp.bk, tp.tiles_s, tp.tiles_o,
                 tp.ksplit, tp.grid, tp.block, tp.ws_bytes);
    }
    return WQ_OK;
}

} // extern "C"
