/*
 * wqmm.h — C ABI of libwqmm.so, the weight-resident quantized matmul for
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四, the
 * qmatmul.comp header; colibri-analysis "CUDA 后端", section 1, quant_matmul):
 *
 *     y[s,o] = scale[o] * sum_{i<I} dequant(W[o,i]) * x[s,i]
 *
 * W is an [O, I] weight matrix kept resident in device memory in one of four
 * storage formats, with one fp32 scale per output row applied after the sum;
 * x is fp32 [S, I] and y is fp32 [S, O], both row-major with s outer
 * (x[s*I + i], y[s*O + o]).
 *
 * Storage formats (format list: colibri-analysis "CUDA 后端", section 1,
 * row_bytes; codes 0..2 from the Vulkan tensor description in "第 8 章 · 02",
 * section 三; dequant offsets from weight_at in the same section 1):
 *   WQ_F32  4 bytes per element, little-endian IEEE single, used as is;
 *   WQ_I8   1 byte per element, two's complement, used as is;
 *   WQ_I4   2 elements per byte, even element in the low nibble,
 *           value = nibble - 8;
 *   WQ_I2   4 elements per byte, element 4j+k in bits 2k..2k+1 of byte j,
 *           value = code - 2.
 * A packed host row is row_bytes = ceil(I*bits/8) bytes; rows follow each
 * other with no padding; unused high bits of a row's last byte are ignored.
 *
 * Accuracy contract: for every output element,
 *     |y - y_exact| <= 1e-5 * sum_i |scale[o] * q[o,i] * x[s,i]| + 1e-30,
 * and results are deterministic (same inputs, same launch configuration,
 * same bits). Rows whose codes all decode to 0, rows with scale 0 and
 * products that are exact integers sums are reproduced exactly.
 *
 * Errors: every function returns WQ_OK (0) or a negative WQ_E_* code; nothing
 * aborts or exits, and on an error no output is written. A caller that gets
 * an error may fall back to its own CPU path, as the reference engine does
 * when its GPU call fails (colibri-analysis "CUDA 后端", section 3.1).
 *
 * Threads: calls on one device must not overlap from several host threads.
 * Calls on different devices are independent.
 */
#ifndef WQMM_H
#define WQMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_MAX_DEVICES 16   /* size of the static device table */
#define WQ_GEMV_MAX_S 8     /* largest S the register GEMV serves (by default f32 only; quantized formats take it at S = 1 and the matrix-core paths above) */

enum wq_fmt { WQ_F32 = 0, WQ_I8 = 1, WQ_I4 = 2, WQ_I2 = 3 };

enum wq_status {
    WQ_OK = 0,
    WQ_E_INVAL = -1,       /* bad argument (NULL pointer, size, format, device list) */
    WQ_E_NODEV = -2,       /* no usable GPU, or the device is not gfx950-capable */
    WQ_E_NOTINIT = -3,     /* device not opened by wq_init */
    WQ_E_OOM = -4,         /* device memory (or WQ_MEM_LIMIT_BYTES budget) exhausted */
    WQ_E_MISMATCH = -5,    /* re-upload with a different device/format/shape */
    WQ_E_HIP = -6,         /* the HIP runtime reported an error */
    WQ_E_FAULT = -7,       /* failure injected with WQ_FAULT (tests of caller fallback) */
    WQ_E_UNSUPPORTED = -8  /* valid request this build cannot serve */
};

typedef struct wq_tensor wq_tensor; /* opaque resident weight tensor */
typedef struct wq_group wq_group;   /* opaque set of tensors run in one launch */

/*
 * Open devices (colibri-analysis "CUDA 后端", section 1, coli_cuda_init: the
 * ordinals are validated and each GPU gets its own context).
 * devices: host array of ndev ordinals; NULL with ndev == 0 opens device 0.
 * Rejects duplicates, negative or out-of-range ordinals and ndev >
 * WQ_MAX_DEVICES (WQ_E_INVAL); no GPU or a non-gfx950 GPU gives WQ_E_NODEV.
 * Calling it again is allowed: already-open devices are kept, and the
 * environment knobs are read again (WQ_FORCE_PATH=gemv|tiled|skinny|auto,
 * WQ_GEMV_MAX_S, WQ_MEM_LIMIT_BYTES, WQ_FAULT=upload|launch,
 * WQ_SKINNY_RING=4|6 (chunks of loads in flight per wave of the few-rows
 * kernel, capped at its spill-free depth; default 2), WQ_WAVES_PER_CU,
 * WQ_TILED_MODE=bf16x3|bf16|fp32, WQ_TILED_SHAPE=BMxBNxBK (a compiled tile shape:
 * 128x96x64, 128x96x128, 64x64x64, 64x64x128, 64x192x64 or 16x128x64 in the
 * bf16x3 mode, the same but 16x128x64 in the bf16 mode, 128x96x32 or 64x64x32
 * in fp32 mode; a 128-deep shape is taken with group scales only when the
 * group size is a multiple of 128, else the automatic choice stands),
 * where WQ_TILED_MODE=bf16 is an opt-in reduced-precision tiled mode for
 * quantized weights (the int4 x 16-bit-activation matrix-unit dispatch in
 * colibri docs "CUDA backend (Linux)", section "The GPU-resident pipeline"):
 * each activation is rounded
 * to the nearest bf16 (ties to even) and multiplied once on the bf16 matrix
 * units. Its results are within the usual bound of the exact product on the
 * rounded activations, hence within 2^-8 * sum_i |scale * q * x| of the exact
 * product on the fp32 ones; the default bf16x3 mode gives up no precision.
 * It applies to calls that take the tiled path only (quantized S > 32 by
 * default),
 * WQ_VERBOSE=1 prints one line per device on stderr).
 */
int wq_init(const int *devices, int ndev);

/*
 * Free and total device memory in bytes (colibri-analysis "CUDA 后端",
 * section 1, coli_cuda_mem_info). free_b/total_b: host pointers, either may be
 * NULL. WQ_E_NOTINIT if the device was not opened.
 */
int wq_mem_info(int device, size_t *free_b, size_t *total_b);

/* Bytes of one packed host row: ceil(I*bits/8); -1 for a bad fmt or I < 0.
 * Host-only, needs no device. */
long wq_row_bytes(int fmt, long I);

/*
 * Upload a weight tensor once and keep it resident (colibri-analysis
 * "CUDA 后端", section 1, coli_cuda_tensor_upload; uploads happen lazily and
 * once, colibri docs "CUDA backend (Linux)", introduction).
 *   t:      in/out handle. *t == NULL: allocate, copy w and scales, set *t.
 *           *t != NULL: nothing is copied; the call only checks that device,
 *           fmt, O and I match the resident tensor (WQ_E_MISMATCH if not).
 *   w:      host pointer to O packed rows of wq_row_bytes(fmt, I) bytes.
 *   scales: host pointer to O floats; may be NULL only for WQ_F32 (scale 1).
 * The copy is synchronous: the caller may free w and scales on return. The
 * library owns the device copy until wq_tensor_free.
 * Errors: WQ_E_INVAL (NULL t or w, bad fmt, O <= 0, I <= 0, missing scales),
 * WQ_E_NOTINIT, WQ_E_OOM, WQ_E_HIP, WQ_E_FAULT (WQ_FAULT=upload).
 */
int wq_tensor_upload(wq_tensor **t, int device, int fmt, int O, int I, const void *w,
                     const float *scales);

/*
 * Upload with group-wise scales: one fp32 scale per (output row o, group of
 * gs consecutive columns) — the group-size field of the Vulkan tensor
 * description (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 三):
 *     y[s,o] = sum_g scales[o*ng + g] * sum_{i in [g*gs, (g+1)*gs)} q[o,i] x[s,i],
 * ng = ceil(I/gs) (the last group may be shorter).
 *   scales: host pointer to O * ng floats, row-major (required).
 *   gs:     group size, a positive multiple of 64 (WQ_E_UNSUPPORTED otherwise;
 *           each 16-byte weight slot and each 64-column tiled step then lies
 *           inside one group). 2 <= S <= 16 runs on the few-rows matrix-core
 *           kernel when gs is a multiple of 128 (int8, int4) or 256 (int2),
 *           else on the tiled path (wq_describe_plan_gs tells which).
 * Formats int8/int4/int2 only (WQ_E_INVAL for WQ_F32 or gs <= 0). Otherwise
 * as wq_tensor_upload; a re-upload also checks gs (WQ_E_MISMATCH). The
 * tensor then works with every matmul call; groups containing such tensors
 * take the grouped few-rows launch (below) when its conditions hold, else
 * one launch per tensor.
 */
int wq_tensor_upload_gs(wq_tensor **t, int device, int fmt, int O, int I, int gs, const void *w,
                        const float *scales);

/*
 * Lazy upload plus a synchronous matmul on host buffers (colibri-analysis
 * "CUDA 后端", section 1, coli_cuda_matmul: upload on first use, copy x in,
 * run, copy y back, all blocking).
 * Same tensor arguments as wq_tensor_upload; x: host [S, I] floats, y: host
 * [S, O] floats (written). S == 0 uploads (if needed) and returns WQ_OK.
 */
int wq_matmul(wq_tensor **t, int device, int fmt, int O, int I, const void *w,
              const float *scales, const float *x, int S, float *y);

/* Synchronous matmul with an already-resident tensor; x, y host pointers.
 * x and y pass through pinned host buffers mapped into the device's address
 * space (library-owned, grown to the largest call, held until the process
 * ends), which kernels on the library stream copy to and from device memory;
 * y is written only when the call succeeds. */
int wq_matmul_t(const wq_tensor *t, const float *x, int S, float *y);

/*
 * Stream-ordered matmul on device buffers, queued on hip_stream (a
 * hipStream_t; NULL = the device's null stream): no copies and no host
 * synchronisation. x_dev: device [S, I] floats, y_dev: device [S, O] floats,
 * both on the tensor's device and 4-byte aligned. The call returns once the
 * work is queued; y_dev is valid after the stream reaches it.
 * Quantized formats at S = 1, f32 at S <= 8: the register GEMV, one kernel
 * launch, no workspace. Quantized 2 <= S <= 32 with I % 4 == 0 and x_dev
 * 16-byte aligned: the few-rows matrix-core kernel, one launch, no
 * workspace (above S = 16 with four waves per block, one block per CU; for
 * S > 20 only where at most one block per CU covers all O rows, else the
 * tiled path). Larger S (or rows the few-rows kernel cannot read in 16-byte
 * runs) with a quantized format (tiled path, bf16x3 mode): two launches that use the
 * stream's workspace (3 * round_up(S, 128) * round_up(fields per row, 128)
 * bf16 values, 16-row padding for S <= 16; when K is split across blocks,
 * a third launch adds ksplit * S * O fp32 partials kept after them;
 * wq_describe_plan prints the size). Each stream has a workspace of its
 * own, so tiled calls on different streams may overlap; it grows on demand,
 * which waits for the device to go idle and allocates. Up to 8 streams per
 * device hold one; the first tiled call on a ninth stream takes over the
 * least recently used stream's workspace (also waiting for the device). The
 * key is the stream handle: a destroyed stream's workspace passes to a new
 * stream that gets the same handle, so let a stream's queued calls finish
 * before destroying it. A call being captured into a HIP graph never waits
 * or allocates: it uses its stream's workspace if that is large enough,
 * else the largest workspace on the device that is (the graph then shares
 * that stream's buffer: do not replay it while that stream runs tiled
 * calls), else it returns WQ_E_UNSUPPORTED; so run the largest S once,
 * eagerly, before capturing.
 */
int wq_matmul_dev(const wq_tensor *t, const float *x_dev, int S, float *y_dev, void *hip_stream);

/*
 * wq_matmul_dev for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results as wq_matmul_dev (bit for bit), but
 * the call never allocates or frees anything: the tiled path's workspace is
 * a fixed device array of WQ_NOALLOC_SCRATCH_BYTES per device, reserved for
 * this call when the library is loaded and held until the process ends (its
 * address is looked up in wq_init). A call whose workspace would exceed it
 * (wq_describe_plan prints the size; e.g. S = 2048 with I = 8192 int8)
 * returns WQ_E_UNSUPPORTED before any launch. Every call on a device shares
 * that device's array, which keeps the last call's contents (each call
 * rewrites every part it reads, so nothing needs clearing): calls that
 * overlap in time on one device -- from two streams, or two host threads --
 * race on it and must not be issued. Calls on different devices do not
 * share it. Errors as wq_matmul_dev, plus WQ_E_UNSUPPORTED.
 */
#define WQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int wq_matmul_dev_noalloc(const wq_tensor *t, const float *x_dev, int S, float *y_dev, void *hip_stream);

/* Size in bytes of the fixed device array wq_matmul_dev_noalloc uses. Host-only. */
size_t wq_noalloc_scratch_bytes(void);

/*
 * Build a group of G resident tensors that run together in one launch (the
 * grouped expert matmul of a mixture-of-experts decode step; grouped expert
 * handling at prefill is described in colibri docs "CUDA backend (Linux)",
 * section "The GPU-resident pipeline"). All tensors must be on the same
 * device and share one format. The work split (balanced by weight bytes) is
 * built once here and kept on the device. The group references the tensors:
 * free the group before any of its tensors.
 */
int wq_grouped_create(wq_tensor *const *ts, int G, wq_group **group);

/*
 * Run every tensor of a plain group (a gated group gives WQ_E_INVAL):
 * y_dev[g] = matmul(ts[g], x_dev[g], S[g]).
 * x_dev, S, y_dev: host arrays of G entries (device pointers inside);
 * S[g] == 0 skips tensor g. When every S[g] <= the grouped GEMV limit
 * (4 for int4 and int2, 8 for int8 and f32) and every row
 * fits one wave of the register GEMV, up to 64 tensors run as ONE launch on
 * hip_stream whatever their shapes (e.g. the gate, up and down projections
 * of 8 experts: 24 tensors with 3 KiB and 1 KiB rows), the work cut into
 * pieces of equal weight bytes when the group is created; more tensors take
 * one launch per 64 (none of this with group-wise scales). Otherwise, when
 * every S[g] <= 32 (16 with group-wise scales), every x_dev[g] is 16-byte
 * aligned, every I % 4 == 0 and every group size is a multiple of 128
 * (int8, int4) or 256 (int2), the
 * tensors run on the few-rows matrix-core kernel, one launch per 32 tensors
 * with S[g] > 0 (blocks of 16 to 64 output rows of one tensor each; the
 * tile is that of the largest S[g]; with any group-scaled tensor the
 * group-scaled kernel, where a row-scaled tensor is one group as long as
 * its row). Otherwise one wq_matmul_dev per
 * tensor, still stream-ordered (the tiled ones share the stream's
 * workspace, in stream order).
 */
int wq_grouped_matmul_dev(wq_group *group, const float *const *x_dev, const int *S,
                          float *const *y_dev, void *hip_stream);

/* Release a group (plain or gated); NULL is a no-op. */
int wq_grouped_free(wq_group *group);

/*
 * Gated feed-forward of a mixture-of-experts layer (the fused gate/up matmul
 * feeding the down projection: the gated up-projection shader
 * qmatmul_gate_up.comp named in colibri "第 8 章 · 02 CUDA/Metal/Vulkan
 * 三后端", learning goals and section recap, whose body and activation the
 * pages do not give; SiLU gating is the reading taken). For expert e:
 *
 *     g = gate_e . x_e,  u = up_e . x_e      (each as wq_matmul_dev computes it)
 *     h_e[s,o] = silu(g[s,o]) * u[s,o],      silu(z) = z / (1 + e^-z)
 *     y_e = down_e . h_e
 *
 * wq_swiglu_create pairs gate[e] with up[e] (host arrays of E tensors, all on
 * one device in one format; gate[e] and up[e] must have the same O, I and
 * group size, else WQ_E_INVAL) into a gated group, freed with
 * wq_grouped_free before its tensors. The group references the tensors.
 *
 * wq_swiglu_matmul_dev: h_dev[e] = h_e, an fp32 [S[e], O_e] device buffer,
 * for x_dev[e] fp32 [S[e], I_e] (host arrays of E device pointers; S[e] == 0
 * skips expert e). Stream-ordered on hip_stream. With every S[e] within the
 * grouped GEMV limit, one scale per row and rows that fit one wave, all experts run
 * in one launch that reads each gate row and up row once and writes h
 * directly (g and u never reach memory); otherwise, on the conditions of
 * the grouped few-rows launch (see wq_grouped_matmul_dev), the gate and up
 * matmuls of up to 16 experts run per launch of the few-rows matrix-core
 * kernel (gate -> h_dev[e], up -> the stream's workspace), then one
 * activation launch per 32 experts; otherwise each expert runs as its own
 * paired launch, or (S above the grouped GEMV limit, or group-wise scales)
 * as gate -> h_dev[e], up -> the stream's workspace, then an activation
 * kernel. The forms through the workspace may grow it (not while the stream
 * is being captured: see wq_matmul_dev; warm up first).
 *
 * Accuracy: g and u meet the matmul contract; h is silu and the product
 * evaluated in fp32 on those values (a few ulps, no further cancellation).
 *
 * wq_swiglu_ffn_dev: the whole layer, both launches stream-ordered on
 * hip_stream: h_dev as above (the caller's intermediate buffers), then
 * y_dev[e] = down_e . h_e through the plain group `down` (wq_grouped_create
 * of the E down tensors, down[e]->I == gate[e]->O, else WQ_E_INVAL);
 * y_dev[e] is fp32 [S[e], O_down_e].
 */
int wq_swiglu_create(wq_tensor *const *gate, wq_tensor *const *up, int E, wq_group **group);
int wq_swiglu_matmul_dev(wq_group *gated, const float *const *x_dev, const int *S,
                         float *const *h_dev, void *hip_stream);
int wq_swiglu_ffn_dev(wq_group *gated, wq_group *down, const float *const *x_dev, const int *S,
                      float *const *h_dev, float *const *y_dev, void *hip_stream);

/* Release a resident tensor (colibri-analysis "CUDA 后端", section 1,
 * coli_cuda_tensor_free). NULL is a no-op. */
int wq_tensor_free(wq_tensor *t);

/* Static description of a status code; never NULL. */
const char *wq_strerror(int code);

/*
 * Introspection for tests and tools: the kernel path wq_matmul_dev would take
 * for (fmt, O, I, S) on this build, written as a NUL-terminated string into
 * buf (e.g. "gemv fmt=2 smax=1 lw=16 kmax=4 k=3 team=1 d=4 rows_per_team=12 grid=256 block=256",
 * "skinny fmt=2 m=2 rpl=2 nb=3 waves=8 ring=2 chunks=48 chunks_per_wave=6 grid=256 block=512 workspace=0",
 * or "tiled fmt=1 mode=bf16x3 bm=128 bn=96 bk=64 tiles_s=4 tiles_o=64 ksplit=1 grid=256 block=512 workspace=...").
 * Host-only: needs no device. Returns WQ_OK or WQ_E_INVAL.
 */
int wq_describe_plan(int fmt, int O, int I, int S, char *buf, size_t buflen);

/* The same for a tensor uploaded with wq_tensor_upload_gs(..., gs, ...)
 * (gs = 0: as wq_describe_plan). WQ_E_INVAL also for gs < 0. */
int wq_describe_plan_gs(int fmt, int O, int I, int S, int gs, char *buf, size_t buflen);

/*
 * Measurement helper (not part of the matmul): the practical HBM read
 * ceiling. Reads `bytes` (a multiple of 16) from the device buffer buf_dev
 * (16-byte aligned) exactly once with the 128-bit non-temporal loads the
 * GEMV streams its weights with: `waves` waves (a positive multiple of 4,
 * blocks of 4 waves) each read one contiguous chunk, keeping
 * loads_in_flight (1, 2, 4, 5, 8, 9, 12, 16, 18, 24 or 36) loads of 1 KiB in
 * flight.
 * out_dev (device, 4-byte aligned) receives 64 * waves words (an
 * exclusive-or of the words read, so the loads cannot be dropped).
 * Stream-ordered on hip_stream, no host synchronisation. It gives the GEMV
 * timings a measured ceiling to be read against (colibri docs "CUDA backend
 * (Linux)" print no kernel-level rates, so the ceiling is measured, not
 * quoted). Errors: WQ_E_INVAL for a bad argument, WQ_E_HIP.
 */
int wq_stream_read_dev(const void *buf_dev, size_t bytes, int waves, int loads_in_flight, unsigned *out_dev,
                       void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* WQMM_H */
