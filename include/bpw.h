/*
 * bpw.h - C ABI of libbpw: ternary bit-plane (.trit v1) GEMV on AMD Instinct MI355X (gfx950).
 *
 * What is computed. For a ternary matrix W (rows x cols, entries in {-1, 0, +1}) and an int8
 * activation x, each output row is the select-accumulate sum
 *     y[r] = sum of x[c] over W[r][c] = +1  minus  sum of x[c] over W[r][c] = -1
 * ("Tritium: One Weight Format for Ternary Inference on Commodity CPUs and Multiplier-Free
 * Hardware", introduction, Equations 2-3; "The .trit format, version 1", section 1). The sum is
 * exact in int32 and independent of evaluation order (Tritium paper, "CPU kernels" and
 * "Verification"); x is widened before it is negated, so x = -128 is exact (Tritium paper,
 * "The hardware core"). The fp32 output applies the activation scale, then the per-tensor
 * weight scale, each multiply rounded on its own: y = ((float)acc * x_scale) * w_scale
 * (format page 2.3: the dequantised weight is scale * trit; Tritium paper, "Why exactness,
 * concretely": scales are applied in turn, not folded).
 *
 * Weight layout ("The .trit format, version 1", 2.3 "Ternary payload"). beats_per_row
 * (bpr) = ceil(cols / 64). Beat b of row r is the 16 bytes at offset (r * bpr + b) * 16:
 * bytes 0..8 are the little-endian u64 pos plane (bit k set: W[r][64b + k] = +1), bytes 8..16
 * the neg plane (bit k set: W[r][64b + k] = -1). Invariants: P1 pos & neg == 0 in every beat;
 * P2 bits past cols in each row's last beat are clear (Tritium paper, "Invariants"). The
 * library never rewrites these bytes: what is validated is what the GPU streams.
 *
 * Conventions for every entry point:
 *   - Every function that can fail returns bpw_status; nothing is printed, no exception
 *     crosses the ABI. A failing call also records a one-line reason, readable with
 *     bpw_last_error() on the same host thread.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are GPU memory of the
 *     current HIP device (for example a PyTorch tensor's data_ptr()). The library allocates
 *     no device memory: all device buffers, workspaces and streams belong to the caller and
 *     must outlive the work queued on them.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream. Launches are
 *     asynchronous; faults inside a kernel surface at the caller's next synchronisation.
 *   - Only gfx950 runs the kernels. Any other device returns BPW_E_ARCH; there is no slower
 *     fallback path (Tritium paper, "CPU kernels": a pinned kernel that cannot run is an error).
 *   - A shape the kernels cannot serve returns an error; nothing is silently skipped.
 */
#ifndef BPW_H
#define BPW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BPW_ABI_VERSION 1

typedef enum bpw_status {
    BPW_OK = 0,
    BPW_E_INVAL = 1,          /* bad argument: null pointer, negative size, value outside {-1,0,1}, bad scale */
    BPW_E_SIZE = 2,           /* byte length does not match rows * bpr * 16, or a buffer is too small */
    BPW_E_P1_BOTH_BITS = 3,   /* a beat has pos & neg != 0 (format page section 4, check 17) */
    BPW_E_P2_PADDING = 4,     /* a padding bit past cols is set (format page section 4, check 18) */
    BPW_E_NOT_VALIDATED = 5,  /* a device matrix descriptor that bpw_upload did not produce */
    BPW_E_ARCH = 6,           /* the current device is not gfx950 */
    BPW_E_HIP = 7,            /* a HIP runtime call failed (the reason names it) */
    BPW_E_UNSUPPORTED = 8,    /* valid input outside what the kernels serve (the reason says why) */
    BPW_E_FORMAT = 9          /* a .trit container check failed (bpw_trit_err.check names it) */
} bpw_status;

/* Where a validation error sits. Fields not meaningful for the error are -1. */
typedef struct bpw_err {
    int32_t code;  /* a bpw_status */
    int64_t row;   /* offending row */
    int64_t beat;  /* offending beat within the row */
    int64_t col;   /* lowest offending column (P1: the doubly set weight; P2: first set padding bit) */
} bpw_err;

/* A validated host copy of one ternary matrix's planes (library-owned, opaque). */
typedef struct bpw_host_mat bpw_host_mat;

/* A ternary matrix resident on the GPU. Plain data, filled in by bpw_upload only: the `seal`
 * binds the other fields, so a descriptor edited or built by hand is refused with
 * BPW_E_NOT_VALIDATED. The kernels rely on P1 and P2 and carry no per-beat checks. */
typedef struct bpw_dev_mat {
    const void *d_planes; /* device, rows * bpr * 16 bytes, 256-byte aligned */
    int64_t rows;
    int64_t cols;
    int64_t bpr;          /* beats per row = ceil(cols / 64) */
    float w_scale;        /* per-tensor scale, finite and > 0 (format page 2.2) */
    uint32_t reserved;
    uint64_t seal;
} bpw_dev_mat;

/* One batch-1 GEMV of a grouped launch. */
typedef struct bpw_gemv_job {
    bpw_dev_mat m;
    const int8_t *d_x;    /* device int8 activation codes */
    int64_t x_len;        /* bytes readable at d_x; must be >= bpr * 64 (codes past cols are ignored) */
    float x_scale;        /* activation scale: code q stands for x_scale * q */
    uint32_t reserved;
    int32_t *d_out_i32;   /* device int32 [rows]: exact sums */
    float *d_out_f32;     /* device float [rows]: ((float)acc * x_scale) * w_scale, or NULL */
    const float *d_x_scale; /* device float [1] or NULL: if set, the scale is read from here when the
                               kernel runs (for example written by bpw_quantize) and x_scale is ignored */
} bpw_gemv_job;

/* Inner-loop formulation, pinned by name; a pinned kernel that cannot serve the call errors. */
typedef enum bpw_kernel {
    BPW_KERNEL_AUTO = 0,      /* the fastest measured formulation (bit-serial) */
    BPW_KERNEL_BITSERIAL = 1, /* x split into bit planes; per plane one 3-input bit select + popcount
                                 (Tritium paper, "On popcount": the adder-tree formulation) */
    BPW_KERNEL_BYTELANE = 2,  /* each 4-bit mask group widened to byte lanes, then 4-way int8 dot
                                 products (the masked-byte formulation of format page section 1) */
    BPW_KERNEL_MFMA = 3       /* small batch only: planes decoded to int8 weights once per beat, then
                                 16 rows x 64 columns x 16 tokens per v_mfma_i32_16x16x64_i8 */
} bpw_kernel;

/* ------------------------------------------------------------------------ library */

/* BPW_ABI_VERSION of the loaded library. */
int32_t bpw_abi_version(void);

/* Static name of a status code ("BPW_OK", ...); "unknown status" otherwise. */
const char *bpw_status_string(int32_t status);

/* Reason recorded by the last failing call on this host thread ("" if none). Valid until the
 * next failing call on the same thread. */
const char *bpw_last_error(void);

/* BPW_OK if the current HIP device is gfx950, BPW_E_ARCH otherwise (BPW_E_HIP if no device).
 * Every entry point that launches work runs this check first (cached per device). */
bpw_status bpw_device_check(void);

/* ------------------------------------------------------------------------ host: pack / validate / load */

/* Shapes that pack, validate and load accept: 0 <= rows <= INT32_MAX, 0 <= cols <= 2^40 and
 * rows * bpr * 16 < 2^63 (bpr = ceil(cols / 64)); any other shape is BPW_E_INVAL. */

/* Pack row-major int8 trits w [rows x cols] into .trit v1 planes (format page 2.3).
 * planes_len must equal rows * bpr * 16; padding bits are written clear (P2). A value outside
 * {-1, 0, +1} returns BPW_E_INVAL with its row, beat and column in *err (err may be NULL). */
bpw_status bpw_pack_i8(const int8_t *w, int64_t rows, int64_t cols, uint8_t *planes, size_t planes_len,
                       bpw_err *err);

/* Check host planes in O(payload) (format page section 4, checks 15, 17, 18): length, then every
 * beat in row-major order for P1, and each row's last beat for P2 with the 64-bit tail mask. The
 * first offending beat is reported, its lowest bit; within a beat P1 is reported before P2. */
bpw_status bpw_validate(const uint8_t *planes, size_t len, int64_t rows, int64_t cols, bpw_err *err);

/* Copy host planes into a library-owned buffer, validate the copy (as bpw_validate) and check
 * w_scale (finite, > 0: format page 2.2). On success *out owns the copy; free it with
 * bpw_host_mat_free. Later changes to the caller's buffer do not affect a loaded matrix. */
bpw_status bpw_load(const uint8_t *planes, size_t len, int64_t rows, int64_t cols, float w_scale,
                    bpw_host_mat **out, bpw_err *err);

void bpw_host_mat_free(bpw_host_mat *m);

/* Plane bytes of a loaded matrix (rows * bpr * 16); 0 for NULL. */
size_t bpw_host_mat_bytes(const bpw_host_mat *m);

/* ------------------------------------------------------------------------ upload */

/* Copy a loaded matrix's planes byte for byte into caller-owned device memory d_dst (d_len bytes,
 * >= bpw_host_mat_bytes, 256-byte aligned) on `stream`, wait for the copy, and fill *out.
 * The device copy is what later calls read; it must stay allocated and unmodified while *out is
 * used. */
bpw_status bpw_upload(const bpw_host_mat *m, void *d_dst, size_t d_len, void *stream, bpw_dev_mat *out);

/* ------------------------------------------------------------------------ batch-1 GEMV */

/* Device workspace bytes that bpw_gemv / bpw_gemv_plan_create need for these jobs: the job table,
 * the row-group segments of the persistent grid and their per-workgroup offsets. */
size_t bpw_gemv_workspace_bytes(const bpw_gemv_job *jobs, int32_t n_jobs);

/* Run n_jobs independent GEMVs as one kernel launch on `stream`. The job table is copied into d_ws
 * (ws_len >= bpw_gemv_workspace_bytes); this call waits until that copy has landed, so it also
 * waits for earlier work on `stream`. Callers that repeat the same jobs should build a plan once
 * and call bpw_gemv_plan_run. n_jobs == 0 does nothing and returns BPW_OK. Jobs must not write
 * overlapping outputs. */
bpw_status bpw_gemv(const bpw_gemv_job *jobs, int32_t n_jobs, int32_t kernel, void *d_ws, size_t ws_len,
                    void *stream);

/* bpw_gemv without a workspace argument, for callers that cannot allocate device memory (code under
 * graph capture, serving loops, harnesses that forbid hipMalloc). The job and tile tables go into the
 * library's own fixed device array of 1 MiB (one per GPU, held from the first call on that GPU until
 * the process ends); the call allocates no device memory and calls no allocating routine of HIP or
 * torch. The same computation, kernels and results as bpw_gemv, bit for bit. Jobs whose tables need
 * more than 1 MiB (bpw_gemv_workspace_bytes: a decode step's 210 GEMVs need 0.70 MiB) return
 * BPW_E_SIZE and launch nothing. Every call on one GPU rewrites that GPU's array: calls may follow
 * one another on one stream (each waits for its table copy, which is ordered after the previous
 * launch), but calls that overlap on one GPU (other streams, other host threads) race on the tables.
 * Errors as bpw_gemv; n_jobs == 0 does nothing. */
bpw_status bpw_gemv_noalloc(const bpw_gemv_job *jobs, int32_t n_jobs, int32_t kernel, void *stream);

/* A prepared grouped GEMV: the job table already sits in the caller's workspace. */
typedef struct bpw_gemv_plan bpw_gemv_plan;

/* Check the jobs, write their tables into d_ws (waiting for the copy, as bpw_gemv does) and return
 * a host handle. The workspace, the matrices, activations and outputs named by the jobs must stay
 * valid for the plan's lifetime; their contents may change between runs (each run reads the
 * activations as they are when it executes). */
bpw_status bpw_gemv_plan_create(const bpw_gemv_job *jobs, int32_t n_jobs, int32_t kernel, void *d_ws,
                                size_t ws_len, void *stream, bpw_gemv_plan **out);

/* Queue one execution of a plan on `stream`: a single kernel launch, no host-device copies, no
 * writes to the workspace (runs of one plan on different streams only race on the outputs). */
bpw_status bpw_gemv_plan_run(const bpw_gemv_plan *plan, void *stream);

void bpw_gemv_plan_free(bpw_gemv_plan *plan);

/* ------------------------------------------------------------------------ IntMlp gate/up pairs */

/* The gate and up projections of one MLP with the IntMlp epilogue fused in ("Tritium ...",
 * "Numerics", IntMlp): the squared-ReLU stage never becomes floating point. Both projections read
 * the same activation codes x (so they share its scale); with exact row sums a_g, a_u and the
 * uniform positive scales S_g = x_scale * gate.w_scale, S_u = x_scale * up.w_scale,
 *   relu(a_g S_g)^2 (a_u S_u) = t K,   t = relu(a_g)^2 * a_u (int64),   K = S_g^2 * S_u,
 * K computed once in float64 as (S_g * S_g) * S_u with S = (double)x_scale * (double)w_scale.
 * |a| <= 128 * cols, so t is exact in int64 for cols <= 16383 (|t| < 2^55 at 2560 columns); wider
 * pairs are refused with BPW_E_UNSUPPORTED. Outputs must not overlap those of other jobs. */
typedef struct bpw_intmlp_job {
    bpw_dev_mat gate;       /* gate projection */
    bpw_dev_mat up;         /* up projection: same rows and cols as gate */
    const int8_t *d_x;      /* device int8 codes both projections read, 16-byte aligned */
    int64_t x_len;          /* bytes readable at d_x; >= bpr * 64 */
    float x_scale;          /* activation scale (ignored if d_x_scale is set) */
    uint32_t reserved;
    const float *d_x_scale; /* device float [1] or NULL, as in bpw_gemv_job */
    int64_t *d_t;           /* device int64 [rows], 8-byte aligned: t */
    double *d_k;            /* device double [1], 8-byte aligned: K */
    int32_t *d_gate_i32;    /* device int32 [rows] or NULL: a_g */
    int32_t *d_up_i32;      /* device int32 [rows] or NULL: a_u */
} bpw_intmlp_job;

/* Device workspace bytes for a plan over n_jobs plain GEMVs and n_mlp gate/up pairs. */
size_t bpw_gemv_intmlp_workspace_bytes(const bpw_gemv_job *jobs, int32_t n_jobs, const bpw_intmlp_job *mlp,
                                       int32_t n_mlp);

/* As bpw_gemv_plan_create, with gate/up pairs beside the plain jobs: bpw_gemv_plan_run then runs
 * all of them in one kernel launch. Each pair is one job of the launch whose tiles stream the same
 * rows of both matrices and write t (and K, once) instead of the two projections' outputs; a pair
 * with no rows writes nothing, K included. Pairs
 * need the bit-serial kernel (AUTO or BPW_KERNEL_BITSERIAL); BPW_KERNEL_BYTELANE with n_mlp > 0 is
 * BPW_E_UNSUPPORTED. Errors as bpw_gemv_plan_create, plus BPW_E_INVAL for a pair whose matrices
 * differ in shape or whose d_t / d_k is NULL or misaligned. */
bpw_status bpw_gemv_intmlp_plan_create(const bpw_gemv_job *jobs, int32_t n_jobs, const bpw_intmlp_job *mlp,
                                       int32_t n_mlp, int32_t kernel, void *d_ws, size_t ws_len, void *stream,
                                       bpw_gemv_plan **out);

/* ------------------------------------------------------------------------ activation quantiser */

/* One activation to quantise in the Folded mode ("Tritium ...", "Numerics"): int8 codes are taken
 * from u = h * g (the residual stream times the RMS-norm gain) and 1/rms moves into the scale:
 *   m = max |u_i|, q_i = rint((127 * u_i) / m) in float32 (ties to even),
 *   scale = (float)((m / 127) / sqrt(sum_i h_i^2 / n + eps)) with the sum and root in float64.
 * In exact arithmetic these are the codes and scale of quantising the materialised norm
 * (h / rms) * g; the scale is what a GEMV epilogue multiplies by (bpw_gemv_job.d_x_scale). */
typedef struct bpw_quant_job {
    const float *d_h;     /* device float [n]: residual stream */
    const float *d_g;     /* device float [n]: RMS-norm gain */
    int64_t n;            /* elements, >= 1 */
    int8_t *d_q;          /* device int8 [q_len]: codes; bytes n .. q_len-1 are written 0 */
    int64_t q_len;        /* >= n */
    float *d_scale;       /* device float [1]: the scale */
    float eps;            /* the norm's epsilon, finite and >= 0 */
    uint32_t reserved;
} bpw_quant_job;

/* Device workspace bytes bpw_quantize / bpw_quant_plan_create need for n_jobs jobs. */
size_t bpw_quantize_workspace_bytes(int32_t n_jobs);

/* Quantise n_jobs activations, one launch on `stream`. The job table is copied into d_ws
 * (256-byte aligned, ws_len >= bpw_quantize_workspace_bytes); the call waits for that copy.
 * n_jobs == 0 does nothing. Jobs must not write overlapping outputs. */
bpw_status bpw_quantize(const bpw_quant_job *jobs, int32_t n_jobs, void *d_ws, size_t ws_len, void *stream);

typedef struct bpw_quant_plan bpw_quant_plan;

/* The job table written once into d_ws (which, with the jobs' buffers, must outlive the plan);
 * each run is one launch that reads the inputs as they are when it executes. */
bpw_status bpw_quant_plan_create(const bpw_quant_job *jobs, int32_t n_jobs, void *d_ws, size_t ws_len,
                                 void *stream, bpw_quant_plan **out);
bpw_status bpw_quant_plan_run(const bpw_quant_plan *plan, void *stream);
void bpw_quant_plan_free(bpw_quant_plan *plan);

/* ------------------------------------------------------------------------ small-batch GEMM */

/* out[t][r] = sum_c W[r][c] * X[t][c] for t < batch, one kernel launch: each beat is read from HBM once
 * and applied to every token (tokens beyond a workgroup's group re-read it from the cache). X is
 * device int8, token-major, row t at d_X + t * ldx with ldx >= bpr * 64, ldx % 16 == 0 and d_X
 * 16-byte aligned (codes past cols are ignored); (batch + 16) * ldx must stay below 2^32 bytes.
 * x_scales is a HOST float[batch]. d_out_i32 is device int32 [batch x rows]; d_out_f32 (device float
 * [batch x rows], or NULL) gets ((float)acc * x_scales[t]) * w_scale. 1 <= batch <= 64. kernel:
 * BPW_KERNEL_BITSERIAL (select per token), BPW_KERNEL_MFMA (int8 matrix cores), or BPW_KERNEL_AUTO
 * (the faster measured one for the batch); BPW_KERNEL_BYTELANE is refused. Every kernel gives the
 * same integers; with batch == 1 they equal bpw_gemv's bit for bit. Needs no workspace. */
bpw_status bpw_gemm_small_batch(const bpw_dev_mat *m, const int8_t *d_X, int32_t batch, int64_t ldx,
                                const float *x_scales, int32_t *d_out_i32, float *d_out_f32, int32_t kernel,
                                void *stream);

/* Several small-batch calls in one launch (the same computation as bpw_gemm_small_batch per job,
 * each beat decoded once per 16 tokens). All jobs of a plan share the batch size; their X, ldx and
 * outputs follow the rules of bpw_gemm_small_batch. */
typedef struct bpw_sb_job {
    bpw_dev_mat m;
    const int8_t *d_X;      /* device int8 [batch][ldx], 16-byte aligned, ldx % 16 == 0, ldx >= bpr * 64 */
    int64_t ldx;
    const float *x_scales;  /* host float [batch]: copied when the plan is made */
    int32_t *d_out_i32;     /* device int32 [batch][rows] */
    float *d_out_f32;       /* device float [batch][rows] or NULL */
} bpw_sb_job;

typedef struct bpw_sb_plan bpw_sb_plan;

/* Device workspace bytes of a plan over these jobs at this batch size (0 if n_jobs <= 0). */
size_t bpw_gemm_small_batch_workspace_bytes(const bpw_sb_job *jobs, int32_t n_jobs, int32_t batch);

/* Check the jobs, write the job and tile tables into d_ws (256-byte aligned; the call waits for the
 * copy) and return a plan; bpw_gemm_small_batch_plan_run then queues the work for all of them as one
 * launch. The workspace holds the tables only and is not written by a run.
 * Kernels: BPW_KERNEL_MFMA, the int8 matrix cores (any batch, any shape); BPW_KERNEL_BITSERIAL, at
 * batch 1 the bit-serial batch-1 grouped GEMV and at batch 2 to 4 the bit-serial token kernel (every
 * beat streamed once and reduced against each token's bit planes), which serves matrices of 2497 to
 * 2560 or 6849 to 6912 columns only (else BPW_E_UNSUPPORTED); BPW_KERNEL_AUTO picks the batch-1 GEMV
 * at batch 1 and the matrix cores otherwise. All give the same integers and floats, bit for bit. Other
 * kernels are BPW_E_UNSUPPORTED. 1 <= batch <= 64.
 * The X buffers are read as they are when a run executes; the scales are the ones given here. The
 * workspace, matrices, X and outputs must outlive the plan; outputs of different jobs must not
 * overlap. */
bpw_status bpw_gemm_small_batch_plan_create(const bpw_sb_job *jobs, int32_t n_jobs, int32_t batch, int32_t kernel,
                                            void *d_ws, size_t ws_len, void *stream, bpw_sb_plan **out);
bpw_status bpw_gemm_small_batch_plan_run(const bpw_sb_plan *plan, void *stream);
void bpw_gemm_small_batch_plan_free(bpw_sb_plan *plan);

/* ------------------------------------------------------------------------ .trit v1 container */

/* A .trit v1 container ("The .trit format, version 1"): header, embedded config, tensor table and a
 * 64-byte aligned payload of ternary (.trit v1 planes) and dense (F32, BF16) tensors. Opening runs
 * the header checks 1-16 of its section 4 in O(tensor count); bpw_trit_verify runs checks 17-19
 * (P1, P2 and the payload hash) in O(file size). The file is untrusted input: every failure is a
 * status, none a crash. Fields are read and checked in file order, so the first failure in file
 * order is the one reported. */
typedef struct bpw_trit_file bpw_trit_file;

typedef enum bpw_trit_dtype { BPW_TRIT_F32 = 0, BPW_TRIT_TERNARY = 1, BPW_TRIT_BF16 = 2 } bpw_trit_dtype;

/* Where a container check failed. Fields that do not apply are -1 (check 0 when none failed). */
typedef struct bpw_trit_err {
    int32_t code;    /* a bpw_status: BPW_E_FORMAT, or BPW_E_P1_BOTH_BITS / BPW_E_P2_PADDING */
    int32_t check;   /* the failed check, numbered as in the format page's section 4 (1..19) */
    int64_t offset;  /* file offset of the offending field */
    int64_t tensor;  /* tensor record index */
    int64_t row, beat, col;  /* checks 17 and 18: first offending row, beat and column */
} bpw_trit_err;

/* One tensor of an opened container. name and data point into the caller's file bytes. */
typedef struct bpw_trit_tensor {
    const char *name;      /* UTF-8, name_len bytes, not NUL-terminated */
    int64_t name_len;
    int32_t dtype;         /* bpw_trit_dtype */
    int32_t ndim;          /* 1..4 */
    uint32_t dims[4];      /* outermost first; a ternary tensor is rows = dims[0], cols = dims[1] */
    float scale;           /* finite, > 0 */
    uint32_t reserved;
    uint64_t offset;       /* from the payload start, a multiple of 64 */
    uint64_t byte_len;
    const uint8_t *data;   /* the tensor's bytes inside the file */
} bpw_trit_tensor;

/* Open a container held in host memory (for example a mapped file) and run checks 1-16. The handle
 * borrows `bytes`, which must stay unchanged and alive until bpw_trit_close. err may be NULL. */
bpw_status bpw_trit_open(const uint8_t *bytes, size_t len, bpw_trit_file **out, bpw_trit_err *err);
/* Checks 17 (P1) and 18 (P2) on every ternary tensor in record order, then 19 (FNV-1a-64 of the
 * bytes from the payload start to the end of the file against the stored hash) when check_hash is
 * nonzero and a hash is stored (0 = absent). */
bpw_status bpw_trit_verify(const bpw_trit_file *f, int32_t check_hash, bpw_trit_err *err);
void bpw_trit_close(bpw_trit_file *f);
int64_t bpw_trit_tensor_count(const bpw_trit_file *f);
bpw_status bpw_trit_tensor_info(const bpw_trit_file *f, int64_t index, bpw_trit_tensor *out);
/* Index of the tensor with this name, or -1. */
int64_t bpw_trit_find(const bpw_trit_file *f, const char *name, size_t name_len);
/* The embedded config (UTF-8 JSON as stored) and the stored payload hash (0 = absent). */
bpw_status bpw_trit_config(const bpw_trit_file *f, const char **json, size_t *len);
uint64_t bpw_trit_stored_hash(const bpw_trit_file *f);
/* FNV-1a, 64-bit, of len bytes (the container's payload hash). */
uint64_t bpw_fnv1a64(const uint8_t *data, size_t len);
/* A ternary tensor of an opened container as a host matrix, ready for bpw_upload: its planes are
 * copied and validated exactly as bpw_load does (P1, P2), with the record's scale as w_scale. */
bpw_status bpw_trit_load(const bpw_trit_file *f, int64_t index, bpw_host_mat **out, bpw_err *err);

/* One tensor for bpw_trit_write. The caller keeps name and data alive during the call. */
typedef struct bpw_trit_tensor_in {
    const char *name;      /* UTF-8, name_len bytes (1..1024), unique within the file */
    int64_t name_len;
    int32_t dtype;         /* bpw_trit_dtype */
    int32_t ndim;          /* 1..4; a ternary tensor has 2: rows = dims[0], cols = dims[1] */
    uint32_t dims[4];      /* outermost first; entries past ndim are ignored */
    float scale;           /* finite, > 0 (w_scale of a ternary tensor) */
    uint32_t reserved;     /* 0 */
    const uint8_t *data;   /* byte_len bytes: .trit v1 planes (rows * beats_per_row * 16) for a ternary
                              tensor, little-endian elements (product of dims x 4 or 2) for F32 / BF16 */
    uint64_t byte_len;
} bpw_trit_tensor_in;

/* Bytes of the container bpw_trit_write makes from these tensors and a config of config_len bytes.
 * The same field checks as bpw_trit_write except the payload scan; on failure *bytes is 0. */
bpw_status bpw_trit_write_size(const bpw_trit_tensor_in *tensors, int64_t n, size_t config_len, uint64_t *bytes,
                               bpw_trit_err *err);
/* Write a .trit v1 container ("The .trit format, version 1", sections 2-2.4) into out: the header
 * (version 1, no flags), the config, one record per tensor sorted by name (bytewise, so a conversion
 * gives the same bytes whatever the order of the input), each payload at the next multiple of 64
 * after the previous one, the payload starting at the first multiple of 64 after the table and the
 * file ending with the last tensor's bytes; gaps are zero. with_hash != 0 stores the FNV-1a-64 of the
 * payload (every byte from its start to the end of the file), 0 stores no hash. Every field is checked
 * before anything is written, and a tensor a reader would refuse is refused here with the number of
 * the check it would fail (err->check: 6 config, 7 count / names, 8 dtype / ndim / reserved, 9 shape
 * overflow, 10 scale, 14-16 byte_len, 17 / 18 P1 / P2 of a ternary payload with its row, beat and
 * column; err->tensor is the index in `tensors`). out_len below the container's size: BPW_E_SIZE
 * with *written set to the size needed and nothing written. On success *written is the size. Any file
 * it writes opens and verifies with bpw_trit_open and bpw_trit_verify. */
bpw_status bpw_trit_write(const bpw_trit_tensor_in *tensors, int64_t n, const char *config, size_t config_len,
                          int32_t with_hash, uint8_t *out, size_t out_len, uint64_t *written, bpw_trit_err *err);

/* ------------------------------------------------------------------------ BITCOS */

/* BITCOS ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A bitmap and a sign"): a
 * second, lossless layout of the same ternary matrix. Every weight has a presence bit (nonzero);
 * every nonzero, in column order, a sign bit (set for -1): n + nnz bits, 2 - z bits per weight at
 * zero density z. The layout the kernel reads (the page leaves the blocking open): per row,
 * bpr = ceil(cols / 64) presence words (u64, column c at bit c & 63 of word c >> 6, padding clear),
 * and the row's signs in u32 words from word row_start[r] (the row's k-th nonzero at bit k & 31 of
 * word row_start[r] + (k >> 5)); row_start[rows] is the word count. cols <= 8192. */
typedef struct bpw_bitcos_host bpw_bitcos_host;

/* Pack row-major int8 trits (values outside {-1, 0, +1}: BPW_E_INVAL with the position in *err). */
bpw_status bpw_bitcos_pack_i8(const int8_t *w, int64_t rows, int64_t cols, float w_scale, bpw_bitcos_host **out,
                              bpw_err *err);
/* Re-encode a validated .trit matrix (same trits, same scale). */
bpw_status bpw_bitcos_from_planes(const bpw_host_mat *m, bpw_bitcos_host **out);
void bpw_bitcos_free(bpw_bitcos_host *h);
/* Read-only views of the host arrays: presence [rows * bpr], signs [sign_words], row_start [rows + 1]. */
bpw_status bpw_bitcos_arrays(const bpw_bitcos_host *h, const uint64_t **presence, const uint32_t **signs,
                             const uint32_t **row_start, int64_t *sign_words, int64_t *nnz);
/* Device bytes bpw_bitcos_upload needs (the three arrays, each at a 256-byte boundary). */
size_t bpw_bitcos_device_bytes(const bpw_bitcos_host *h);

/* A BITCOS matrix resident on the GPU, filled in by bpw_bitcos_upload only (sealed like bpw_dev_mat). */
typedef struct bpw_dev_bitcos {
    const void *d_base;      /* presence words, then row_start, then signs */
    int64_t rows, cols, bpr;
    int64_t sign_words;
    uint64_t row_start_off;  /* byte offsets from d_base */
    uint64_t signs_off;
    float w_scale;
    uint32_t reserved;
    uint64_t seal;
} bpw_dev_bitcos;

bpw_status bpw_bitcos_upload(const bpw_bitcos_host *h, void *d_dst, size_t d_len, void *stream, bpw_dev_bitcos *out);

/* One batch-1 GEMV on a BITCOS matrix: the same sums and dequantisation as bpw_gemv_job. */
typedef struct bpw_bitcos_job {
    bpw_dev_bitcos m;
    const int8_t *d_x;   /* device int8 codes, 16-byte aligned, x_len >= bpr * 64 */
    int64_t x_len;
    float x_scale;
    uint32_t reserved;
    int32_t *d_out_i32;  /* device int32 [rows] */
    float *d_out_f32;    /* device float [rows] or NULL */
} bpw_bitcos_job;

typedef struct bpw_bitcos_plan bpw_bitcos_plan;
size_t bpw_bitcos_workspace_bytes(const bpw_bitcos_job *jobs, int32_t n_jobs);
/* Job and tile tables written once into d_ws (256-byte aligned; waits for the copy); each run is one
 * launch over all jobs. */
bpw_status bpw_bitcos_plan_create(const bpw_bitcos_job *jobs, int32_t n_jobs, void *d_ws, size_t ws_len, void *stream,
                                  bpw_bitcos_plan **out);
bpw_status bpw_bitcos_plan_run(const bpw_bitcos_plan *plan, void *stream);
void bpw_bitcos_plan_free(bpw_bitcos_plan *plan);

/* ------------------------------------------------------------------------ dense head */

/* The dense tied LM head at batch 1 (Tritium paper, "Where the bytes are"; format page 2.4):
 * y[v] = sum_h W[v][h] * x[h] with W device bfloat16 [rows x cols] row-major (uint16 bit patterns),
 * x device bfloat16 [cols], y device float [rows], float32 accumulation. Rows must be 16-byte
 * aligned: cols % 8 == 0 and d_w 16-byte aligned. */
bpw_status bpw_dense_head_gemv(const uint16_t *d_w_bf16, int64_t rows, int64_t cols, const uint16_t *d_x_bf16,
                               float *d_y, void *stream);

/* ------------------------------------------------------------------------ measurement helpers */

/* Streaming-read probe (Tritium paper, "Method": achieved bandwidth is divided by a streaming-read
 * probe on the same machine): reads len bytes at d_buf (16-byte aligned, len % 16 == 0) once and
 * writes a data-dependent word to d_sink (device uint32 [1]) so the reads cannot be elided. */
bpw_status bpw_stream_read_probe(const void *d_buf, size_t len, uint32_t *d_sink, void *stream);
/* The same read in one of five shapes (0 is the one bpw_stream_read_probe uses): 0: 256-thread
 * workgroups of 10 buffer loads per lane (40 KiB each); 1: the same with global loads; 2: 512 threads
 * x 8 buffer loads (64 KiB); 3: the same with global loads; 4: 256 threads x 4 buffer loads (16 KiB).
 * Every shape reads each byte once, non-temporal, in XCD-contiguous runs of workgroups; a measured
 * roofline takes the best of them. Another shape, or len above 2^40 bytes: BPW_E_INVAL. */
bpw_status bpw_stream_read_probe_shape(const void *d_buf, size_t len, uint32_t *d_sink, int32_t shape,
                                       void *stream);

/* Read and rewrite len bytes at d_buf (16-byte aligned, len % 16 == 0) so that caches hold none of
 * the bytes a following timed kernel will read (size it above L2 + the 256 MB last-level cache). */
bpw_status bpw_cache_flush(void *d_buf, size_t len, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BPW_H */
