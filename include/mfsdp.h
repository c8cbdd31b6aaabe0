/*
 * mfsdp.h - C ABI of the owner-local Muon + AdamW optimizer step (gfx950).
 *
 * What it computes.  "MatrixFSDP: Communication-Free Matrix Optimizers Under
 * ZeRO-3 Parameter Sharding" (arXiv 2607.05895), Abstract and §1: with
 * owner-shaped sharding, each 2D weight lives whole on one data-parallel
 * rank, so that rank can run Muon's Newton-Schulz on it with no optimizer
 * collective, while tensors that are not matrices are grouped onto tail
 * owners and use AdamW.  The update has to be the one full-matrix Muon
 * gives on the gathered matrix (Abstract; §1).  This
 * library is that owner-local step for one GPU: a table of whole tensors
 * (offsets, shapes, dtypes, roles; the paper's MatrixShard metadata, Abstract)
 * that live in one flat parameter buffer, and one call that updates all of
 * them.
 *
 * Per Muon matrix W (rows x cols), gradient G, momentum M (fp32, or bf16 by
 * hparams.momentum_dtype):
 *   M <- beta*M + G;  U <- G + beta*M (Nesterov) or U <- M;
 *   X <- U / (||U||_F + eps), taken in the wide orientation (tall -> U^T);
 *   ns_steps times: A = X X^T;  B = b*A + c*A*A;  X <- a*X + B*X;
 *   O = X back in W's orientation;
 *   W <- W*(1 - lr*weight_decay) - lr*scale*O,
 *   scale = sqrt(max(1, rows/cols)) (mode 0) or 0.2*sqrt(max(rows, cols)) (mode 1).
 * Per AdamW tail tensor (1-based step t):
 *   m <- b1*m + (1-b1)*g;  v <- b2*v + (1-b2)*g^2;
 *   W <- W*(1 - lr_a*wd_a) - lr_a*(m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps_a).
 * Every stored value is rounded once to its storage type, to nearest-even.
 *
 * Ownership.  The caller allocates every device buffer (params, grads,
 * state, workspace, ns_out).  The library never allocates device memory.
 * A plan is host memory owned by the library until mfsdp_plan_destroy.
 *
 * Errors.  Every function returns mfsdp_status; no C++ exception crosses the
 * boundary and nothing aborts the process.  mfsdp_last_error_message()
 * returns a thread-local description of the last failure on this thread.
 */
#ifndef MFSDP_H
#define MFSDP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mfsdp_status {
    MFSDP_OK = 0,
    MFSDP_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad step, out of range */
    MFSDP_ERR_OVERLAP = 2,            /* two table entries share parameter bytes */
    MFSDP_ERR_MISALIGNED = 3,         /* entry offset not a multiple of 16 bytes */
    MFSDP_ERR_UNSUPPORTED = 4,        /* dtype, role, precision or dimension not supported */
    MFSDP_ERR_WORKSPACE_TOO_SMALL = 5,/* workspace_bytes below mfsdp_plan_workspace_bytes */
    MFSDP_ERR_HIP = 6,                /* a HIP runtime call or kernel launch failed */
    MFSDP_ERR_INTERNAL = 7
} mfsdp_status;

typedef enum mfsdp_dtype {
    MFSDP_F32 = 0,
    MFSDP_BF16 = 1
} mfsdp_dtype;

typedef enum mfsdp_role {
    MFSDP_ROLE_AUTO = 0,   /* Muon iff rows > 1 and cols > 1, else AdamW */
    MFSDP_ROLE_MUON = 1,   /* force Muon (rows >= 1, cols >= 1) */
    MFSDP_ROLE_ADAMW = 2   /* force AdamW */
} mfsdp_role;

/* One whole tensor of the owner buffer (one row of the owner table).
 * offset: byte offset into the params buffer; the grads buffer uses the same
 *         offset.  Must be a multiple of 16.
 * rows, cols: logical shape, row-major.  A 1D tensor of length L is rows=1,
 *         cols=L.  rows*cols == 0 is an empty shard: legal and skipped.
 * dtype:  storage type of both the parameter and its gradient.
 * role:   mfsdp_role. */
typedef struct mfsdp_entry {
    uint64_t offset;
    int64_t rows;
    int64_t cols;
    int32_t dtype;
    int32_t role;
} mfsdp_entry;

/* Hyper-parameters.  Floats are used as the float32 values given. */
typedef struct mfsdp_hparams {
    float lr;                 /* Muon learning rate */
    float weight_decay;       /* Muon decoupled weight decay (multiplied by lr) */
    float momentum;           /* beta */
    int32_t nesterov;         /* 1: U = G + beta*M; 0: U = M */
    int32_t ns_steps;         /* Newton-Schulz iterations, 0..64 */
    float ns_a, ns_b, ns_c;   /* quintic coefficients */
    float ns_eps;             /* added to ||U||_F */
    int32_t lr_scale_mode;    /* 0: sqrt(max(1, rows/cols)); 1: 0.2*sqrt(max(rows, cols)) */
    int32_t ns_precision;     /* 0: bf16 operands, fp32 accumulate; 1: fp32 operands and accumulate */
    float adam_lr;
    float adam_beta1;
    float adam_beta2;
    float adam_eps;
    float adam_weight_decay;
    int32_t momentum_dtype;   /* storage type of the Muon momentum: MFSDP_F32 (0, the default) or
                                 MFSDP_BF16, rounded to nearest-even once per step.  bf16 halves the
                                 momentum's memory, keeping the owner's optimizer state small (the
                                 ZeRO-3-scale memory the MatrixFSDP abstract asks for), and the
                                 momentum pass then moves 8 B per bf16 element instead of 12.  The
                                 AdamW moments stay fp32. */
    int32_t ns_tile_gram;     /* output tile edge of the Newton-Schulz Gram contraction: 0 = chosen by
                                 the planner (256 when the phase has at least 512 tiles of 256, else
                                 128), or 128 or 256 to force it (for tests and tuning; the result
                                 is the same up to fp32 summation order) */
    int32_t ns_tile_poly;     /* the same for the polynomial B = b A + c A A */
    int32_t ns_tile_update;   /* the same for the update X <- a X + B X; a forced edge also turns off
                                 the planner's split of a short last round of 256-tiles into 128-tiles */
    uint32_t guard_bytes;     /* 0 normally.  Otherwise at most 16 MiB: the plan leaves this many
                                 bytes (rounded up to 256) unused after every region it lays out in
                                 the state and in the workspace (mfsdp_plan_regions lists them), so
                                 that a test can fill the gaps with canaries and check after a step
                                 that no kernel wrote outside its regions.  Costs only memory. */
} mfsdp_hparams;

typedef struct mfsdp_plan_s* mfsdp_plan_t;

/* Per-entry layout facts a caller needs to read or seed state. */
typedef struct mfsdp_entry_info {
    int32_t role;             /* resolved: MFSDP_ROLE_MUON, MFSDP_ROLE_ADAMW, or -1 for an empty entry */
    int32_t transposed;       /* Muon: 1 if rows > cols (Newton-Schulz runs on the transpose) */
    int64_t m, n;             /* Muon: oriented shape, m = min(rows, cols) */
    uint64_t state_offset;    /* Muon: momentum (momentum_dtype); AdamW: fp32 first moment (bytes into state) */
    uint64_t state_offset2;   /* AdamW: fp32 second moment (bytes into state); 0 otherwise */
    uint64_t ns_out_offset;   /* Muon: element offset of the fp32 O export in ns_out */
    float lr_scale;           /* Muon: the shape scale applied to lr */
} mfsdp_entry_info;

/* Which caller buffer a plan region lies in. */
#define MFSDP_BUFFER_STATE 0
#define MFSDP_BUFFER_WORKSPACE 1

/* One region the plan lays out in the state or the workspace. */
typedef struct mfsdp_region {
    uint64_t offset;          /* bytes into the buffer */
    uint64_t bytes;           /* bytes the step may read or write there */
    int32_t buffer;           /* MFSDP_BUFFER_STATE or MFSDP_BUFFER_WORKSPACE */
    int32_t entry;            /* table entry it belongs to, -1 for a region shared by all entries */
} mfsdp_region;

/* Step flags. */
#define MFSDP_STEP_DESCRIPTORS_RESIDENT 1u  /* the workspace already holds this plan's
                                               descriptors from an earlier step with the
                                               same workspace pointer; skip the upload */

typedef struct mfsdp_step_args {
    void* params;             /* device, updated in place */
    const void* grads;        /* device, read only; same offsets as params */
    void* state;              /* device, mfsdp_plan_state_bytes, zero-filled before step 1 */
    void* workspace;          /* device, mfsdp_plan_workspace_bytes, 256-byte aligned;
                                 library scratch: the caller must not write it between steps */
    uint64_t workspace_bytes;
    int64_t step;             /* 1-based step count (AdamW bias correction) */
    void* stream;             /* hipStream_t; NULL = the null stream */
    float* ns_out;            /* NULL, or device fp32 [mfsdp_plan_ns_out_elems]: O per Muon entry,
                                 row-major in the entry's own shape, at entry_info.ns_out_offset */
    uint32_t flags;           /* MFSDP_STEP_* */
    void** events;            /* NULL, or n_events hipEvent_t created by the caller: the step
                                 records events[0] after the descriptor upload, events[1] after
                                 the AdamW tail, events[2] after momentum + norm, and for
                                 Newton-Schulz iteration k (1-based) events[3k], events[3k+1],
                                 events[3k+2] after its Gram, polynomial and update launches.
                                 Every event is recorded even when its phase is empty. */
    uint32_t n_events;        /* must be >= mfsdp_plan_num_events when events != NULL */
} mfsdp_step_args;

/* Validate an owner table and lower it to a plan (host only; no HIP call).
 * entries: n rows (may be NULL when n == 0).  param_bytes: size of the params
 * buffer, used for bounds checks.  hp: copied into the plan.
 * Errors: INVALID_ARGUMENT (null pointer, n < 0, negative dim, entry past
 * param_bytes, bad hyper-parameter), OVERLAP, MISALIGNED, UNSUPPORTED (dtype,
 * role, ns_precision, momentum_dtype, an ns_tile_* other than 0, 128 and
 * 256, a dimension above 2^22, a Muon matrix whose padded Newton-Schulz
 * buffer reaches 2 GiB).  *out is set only on success.  The plan depends on
 * its arguments only (no environment variable is read). */
mfsdp_status mfsdp_plan_create(const mfsdp_entry* entries, int64_t n, uint64_t param_bytes,
                               const mfsdp_hparams* hp, mfsdp_plan_t* out);

/* Bytes of optimizer state the plan lays out (momentum for Muon entries, fp32
 * or bf16 by hp->momentum_dtype, then fp32 first and second moments for AdamW
 * entries), each region 256-byte aligned. */
mfsdp_status mfsdp_plan_state_bytes(mfsdp_plan_t plan, uint64_t* bytes);

/* Bytes of device workspace one step needs (descriptors, norm partials,
 * Newton-Schulz buffers). */
mfsdp_status mfsdp_plan_workspace_bytes(mfsdp_plan_t plan, uint64_t* bytes);

/* Number of fp32 elements of the optional ns_out export. */
mfsdp_status mfsdp_plan_ns_out_elems(mfsdp_plan_t plan, uint64_t* elems);

/* Number of phase-boundary events a step records when args->events is set
 * (3 + 3*ns_steps). */
mfsdp_status mfsdp_plan_num_events(mfsdp_plan_t plan, uint32_t* n);

/* Number of table entries and the layout facts of entry i. */
mfsdp_status mfsdp_plan_num_entries(mfsdp_plan_t plan, int64_t* n);
mfsdp_status mfsdp_plan_entry_info(mfsdp_plan_t plan, int64_t i, mfsdp_entry_info* info);

/* One owner step: enqueue every kernel on args->stream and return without
 * synchronising.  Launch failures return MFSDP_ERR_HIP; a fault inside a
 * kernel surfaces at the caller's next synchronisation.  One plan serves one
 * stream at a time; two steps that share a workspace must not overlap.
 * Errors: INVALID_ARGUMENT (null plan or args, null buffer needed by the
 * table, step < 1 with an AdamW entry, misaligned workspace, too few
 * events), WORKSPACE_TOO_SMALL, HIP. */
mfsdp_status mfsdp_owner_step(mfsdp_plan_t plan, const mfsdp_step_args* args);

/* Every region the plan lays out, state first, then workspace, each in
 * increasing offset: Muon momentum and AdamW first and second moments in the
 * state; in the workspace the descriptor blob (one region: it is uploaded
 * as one copy), the per-matrix scale factors, the norm partial sums, and per
 * Muon matrix its two X^T buffers and its A and B.  The step reads and
 * writes state and workspace bytes inside these regions only.  Writes
 * min(*count, capacity) entries to regions (which may be NULL when capacity
 * is 0) and the total number to *count.  Host only.
 * Errors: INVALID_ARGUMENT (NULL plan or count, capacity < 0, NULL regions
 * with capacity > 0). */
mfsdp_status mfsdp_plan_regions(mfsdp_plan_t plan, mfsdp_region* regions, int64_t capacity, int64_t* count);

/* ---- A step that allocates nothing ----
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * step as mfsdp_owner_step (same kernels, bitwise the same results), except
 * that the workspace is a fixed array inside the library: a file-scope
 * device array of MFSDP_STATIC_WORKSPACE_BYTES, which every GPU the library
 * runs on holds until the process ends.  The caller still passes params,
 * grads, state, ns_out and events as for mfsdp_owner_step, with workspace =
 * NULL and workspace_bytes = 0.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); on its first call on a device it
 * looks up that device's copy of the array (hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  The step writes every workspace
 * byte before it reads it, so nothing is cleared between calls.
 * MFSDP_STEP_DESCRIPTORS_RESIDENT skips the descriptor upload only when the
 * previous static call on this device used the same plan.
 * Errors: those of mfsdp_owner_step, plus INVALID_ARGUMENT (workspace not
 * NULL or workspace_bytes not 0), WORKSPACE_TOO_SMALL (the plan needs more
 * than MFSDP_STATIC_WORKSPACE_BYTES: use mfsdp_owner_step), UNSUPPORTED
 * (device index 64 or more), HIP. */
#define MFSDP_STATIC_WORKSPACE_BYTES (64ull << 20)
mfsdp_status mfsdp_owner_step_static(mfsdp_plan_t plan, const mfsdp_step_args* args);

/* Free a plan.  NULL is accepted. */
mfsdp_status mfsdp_plan_destroy(mfsdp_plan_t plan);

/* ---- Owner planner (host only) ----
 *
 * "MatrixFSDP" (arXiv 2607.05895), Abstract: a balance-aware owner planner
 * decides which data-parallel rank owns each whole 2D weight, and tensors
 * that are not matrices are grouped onto a few tail owners.  The pages name the
 * planner only; this one reads "balance-aware" as: every tensor goes whole
 * to one owner, an owner's step time is the sum of its tensors' costs, and
 * the plan minimises the largest owner time under a per-owner memory cap.
 *
 * Cost of a tensor: Muon (m = min(rows, cols), n = max): ns_steps * (4 m^2 n
 * + 2 m^3) / flop_rate + rows*cols * (3 es + 2 em + es_ns) / byte_rate (grad
 * read, param read and write, momentum read and write, the Newton-Schulz
 * input write; es = param bytes, em = momentum bytes (4, or 2 with
 * momentum_dtype MFSDP_BF16), es_ns = 2 for bf16 Newton-Schulz, 4 for fp32);
 * AdamW: rows*cols * (3 es + 16) / byte_rate.
 * Memory of a tensor on its owner: params and grads (2 es per element),
 * state (em B per element for Muon, 8 for AdamW), and for Muon the
 * Newton-Schulz buffers of mfsdp_plan_create (two X^T of n_p x m_p and A, B
 * of m_p x m_p, m_p and n_p padded to 256, es_ns per element), each region
 * rounded up to 256 bytes.  (The plan's descriptor blob and norm partials,
 * a few bytes per tile, are not counted.)
 *
 * Algorithm: tensors in decreasing cost (ties: larger memory, then lower
 * index) each go to the owner with the least cost so far that has room
 * under the cap (ties: lower owner); then moves and swaps of single tensors
 * off the most loaded owner are applied while they lower the largest owner
 * cost.  Deterministic.  Without a binding cap the first pass alone is
 * within 4/3 of the optimal largest cost (longest-processing-time bound).
 */
typedef struct mfsdp_tensor {
    int64_t rows, cols;       /* 1D tensors: rows = 1; rows*cols = 0 is an empty tensor */
    int32_t dtype;            /* mfsdp_dtype of params and grads */
    int32_t role;             /* mfsdp_role, resolved as in mfsdp_entry */
} mfsdp_tensor;

typedef struct mfsdp_partition_params {
    int32_t n_owners;         /* >= 1 */
    int32_t ns_steps;         /* Newton-Schulz iterations in a Muon tensor's cost, >= 0 */
    int32_t ns_precision;     /* 0: bf16 Newton-Schulz buffers, 1: fp32 */
    int32_t momentum_dtype;   /* Muon momentum storage, as in mfsdp_hparams: MFSDP_F32 (0) or MFSDP_BF16 */
    uint64_t mem_cap_bytes;   /* per-owner memory cap; 0 = none */
    double flop_rate;         /* FLOP/s of the Newton-Schulz contractions, > 0 */
    double byte_rate;         /* bytes/s of the elementwise passes, > 0 */
} mfsdp_partition_params;

typedef struct mfsdp_tensor_place {
    int32_t owner;            /* 0 .. n_owners-1 */
    int32_t role;             /* resolved: MFSDP_ROLE_MUON or MFSDP_ROLE_ADAMW (empty tensors: ADAMW) */
    uint64_t offset;          /* bytes into the owner's flat parameter buffer: the owner's tensors in
                                 input order, each at a 256-byte aligned offset */
    double cost;              /* seconds, by the model above */
    uint64_t mem_bytes;       /* by the model above */
} mfsdp_tensor_place;

/* Assign n tensors to owners.  place: n entries, written on success.
 * owner_cost, owner_mem_bytes, owner_param_bytes: NULL or n_owners entries
 * each (sum of costs, sum of memory, end of the last tensor in the owner's
 * flat buffer).  Each owner's tensors, in input order at their offsets, form
 * a table mfsdp_plan_create accepts.
 * Errors: INVALID_ARGUMENT (null pointer, n < 0, n_owners < 1, negative
 * dimension, ns_steps < 0, rates not positive and finite), UNSUPPORTED
 * (dtype, role, ns_precision, a tensor larger than the memory cap, or no
 * owner with room left for a tensor). */
mfsdp_status mfsdp_owner_partition(const mfsdp_tensor* tensors, int64_t n, const mfsdp_partition_params* pp,
                                   mfsdp_tensor_place* place, double* owner_cost, uint64_t* owner_mem_bytes,
                                   uint64_t* owner_param_bytes);

/* ---- Owner-shard checkpoint resharding (host only) ----
 *
 * "MatrixFSDP" (arXiv 2607.05895), Abstract: owner-shard checkpoint
 * resharding.  A checkpoint holds whole tensors; these two calls copy one
 * owner's tensors and their optimizer state between the owner's flat
 * buffers (laid out by its plan) and one buffer per tensor, in host memory,
 * byte for byte (no conversion).  Resharding to another owner count is
 * gather from every old owner, mfsdp_owner_partition for the new count,
 * scatter into every new owner; every value comes back bit-exact.
 *
 * For entry i of the plan's table (numel = rows*cols):
 *   tensors[i]  numel parameter elements in the entry's dtype, row-major;
 *   state1[i]   numel elements: Muon momentum (the plan's momentum_dtype), or AdamW first moment (fp32);
 *   state2[i]   numel fp32: AdamW second moment (unused for Muon).
 * Any array pointer may be NULL (that part is not copied); an element may be
 * NULL where numel is 0 or the part does not apply.  params / state are the
 * owner's buffers (param_bytes >= the end of its last tensor, state_bytes >=
 * mfsdp_plan_state_bytes).  Bytes outside the tensors and state regions are
 * not touched.
 * Errors: INVALID_ARGUMENT (null plan, a needed buffer or element NULL,
 * buffer too small). */
mfsdp_status mfsdp_owner_gather(mfsdp_plan_t plan, const void* params, uint64_t param_bytes, const void* state,
                                uint64_t state_bytes, void* const* tensors, void* const* state1,
                                void* const* state2);
mfsdp_status mfsdp_owner_scatter(mfsdp_plan_t plan, const void* const* tensors, const void* const* state1,
                                 const void* const* state2, void* params, uint64_t param_bytes, void* state,
                                 uint64_t state_bytes);

/* ---- Measurement probes (NOT part of the optimizer step) ----
 *
 * The two calls below compute nothing of the owner step and touch none of
 * a plan's buffers.  They exist so that a benchmark can report, on the
 * same GPU and in the same run, the rates the part sustains for the two
 * kinds of work the step does (bf16 MFMA on Gaussian data; HBM streaming),
 * beside the published peaks.  A caller that only runs the optimizer never
 * needs them. */

/* Measurement support (not part of the step): enqueue on `stream` a
 * register-only loop of bf16 MFMAs (v_mfma_f32_32x32x16_bf16, fp32
 * accumulate) over `blocks` blocks of 4 waves, each wave running `iters`
 * iterations of 32 MFMAs on 16 operand fragments per lane taken from
 * `operands` (device memory, operand_bytes >= 1024, a multiple of 16,
 * 16-byte aligned; read only).  The MFMA clock depends on the operand data,
 * so with the contractions' own kind of data (Gaussian bf16) the elapsed
 * time gives the rate the part sustains for them, as opposed to the
 * published dense peak.  sink: device, blocks * 4 floats, written.  *flops
 * (optional) receives the FLOPs enqueued.  The caller times the launch (for
 * example with events on `stream`).  Errors: INVALID_ARGUMENT, HIP. */
mfsdp_status mfsdp_probe_mfma_bf16(const void* operands, uint64_t operand_bytes, int32_t blocks, int32_t iters,
                                   float* sink, void* stream, double* flops);

/* Measurement support (not part of the step): enqueue on `stream` one pass
 * of 16-byte accesses over `bytes` of device memory: mode 0 reads src, mode
 * 1 writes dst, mode 2 copies src to dst (as many bytes read as written, the
 * mix of the elementwise phases).  2048 blocks of 256 threads, each walking
 * contiguous 32 KB chunks with 8 accesses in flight per thread.  The caller
 * times the launch; the
 * bytes moved are `bytes` (modes 0, 1) or 2 * bytes (mode 2).  sink: device,
 * 8192 floats, written.  Errors: INVALID_ARGUMENT (mode, NULL buffer, bytes
 * not a nonzero multiple of 16, misaligned buffer), HIP. */
mfsdp_status mfsdp_probe_hbm(void* dst, const void* src, uint64_t bytes, int32_t mode, float* sink, void* stream);

/* Static description of a status code. */
const char* mfsdp_status_string(mfsdp_status status);

/* Thread-local description of the last error on this thread ("" if none). */
const char* mfsdp_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* MFSDP_H */
