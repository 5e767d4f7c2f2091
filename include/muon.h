/*
 * muon.h - C ABI of the MI355X (gfx950) Muon per-owner update step.
 *
 * One call of muon_step performs, for every weight matrix of a plan, the Muon
 * update as the pages describe it:
 *   - "DeepSpeed now supports Muon" (setupai.cc), section "technical deep
 *     dive": Newton-Schulz (NS) iterations orthogonalize the momentum-based
 *     update of 2-D weight matrices; weight decay is decoupled; each
 *     parameter's update is scaled so its RMS matches AdamW's, letting AdamW's
 *     lr and wd carry over.
 *   - DMuon announcement (wjxwpt.net), improvement 2 "shape-adaptive execution
 *     stack": per shape the mathematical form (matrix space or m x m Gram
 *     space, item 1), the execution mode (alone or batched with other matrices)
 *     and the kernel change; the step does not change the update rule.
 *   - DMuon announcement (zaocj.com), second of the "three moves": many kernels
 *     are tried on a new shape, the fastest is kept and reused for that shape.
 *
 * Per matrix W (rows x cols), gradient g and fp32 momentum buf:
 *   buf <- beta*buf + g;  d <- g + beta*buf           (Nesterov; plain: d <- buf)
 *   X0  <- d / (||d||_F + eps)
 *   X   <- NS_T(X0): T times  A = X X^T, B = b A + c A^2, X <- a X + B X
 *          (on the smaller side: tall matrices are iterated as their transpose)
 *   W   <- W - lr * (wd * W + s * X),   s = rms_scale * sqrt(max(rows, cols))
 * Both terms of the last line use the old W.  fp32 matrices take an fp32 NS;
 * bf16 matrices take bf16 MFMA operands with fp32 accumulation.
 *
 * Conventions for every entry point:
 *   - returns a muon_status; MUON_OK is 0.  No C++ exception crosses the ABI.
 *     muon_last_error() returns a thread-local message about the last failure.
 *   - "device pointer" means memory on the HIP device that was current when the
 *     plan was created; "host pointer" means ordinary process memory.
 *   - matrices are dense row-major, rows x cols, leading dimension = cols.
 *   - a stream argument is a hipStream_t passed as void* (NULL = null stream).
 *   - graphs the caller captures: muon_step, muon_step_schedule,
 *     muon_orthogonalize and muon_adamw_step keep their per-tensor pointer
 *     tables in device memory and upload a changed table only outside graphs.
 *     A call on a stream under capture must pass the pointers of the plan's
 *     previous call made outside the capture (ESTATE otherwise, nothing
 *     enqueued); the graph reads the table at every replay, so replay it
 *     while the plan's latest call outside graphs used those same pointers.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 13

typedef enum muon_status {
  MUON_OK = 0,
  MUON_EINVAL = 1,        /* bad argument (NULL pointer, negative count, non-finite scalar) */
  MUON_EUNSUPPORTED = 2,  /* unsupported dtype, zero-size matrix, no gfx950 device */
  MUON_ENOMEM = 3,        /* device or pinned-host allocation failed / over the workspace cap */
  MUON_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
  MUON_ESTATE = 5         /* call not valid for this plan (e.g. step on a host-only plan) */
} muon_status;

typedef enum muon_dtype { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

typedef enum muon_precision {
  MUON_PRECISION_AUTO = 0,  /* fp32 NS for fp32 params, bf16 MFMA NS for bf16 params */
  MUON_PRECISION_FP32 = 1,  /* fp32 NS for every matrix */
  MUON_PRECISION_BF16 = 2   /* bf16 MFMA NS for every matrix */
} muon_precision;

typedef enum muon_form {
  MUON_FORM_AUTO = 0,    /* the planner chooses per shape (timed once, or by cost model) */
  MUON_FORM_DIRECT = 1,  /* NS in the m x n matrix space */
  MUON_FORM_GRAM = 2     /* NS recursion in the m x m Gram space, X_T = Q_T X0 */
} muon_form;

typedef enum muon_tune {
  MUON_TUNE_OFF = 0,   /* never time: analytic cost model only (deterministic) */
  MUON_TUNE_ONCE = 1,  /* use the cache; time and record shapes it does not hold */
  MUON_TUNE_FORCE = 2  /* time every shape again and rewrite its cache entries */
} muon_tune;

/* One weight matrix.  The gradient has the parameter's dtype; the momentum is fp32. */
typedef struct muon_matrix_desc {
  int64_t rows;
  int64_t cols;
  int32_t dtype;     /* muon_dtype of the parameter and its gradient */
  int32_t reserved;  /* must be 0 */
} muon_matrix_desc;

typedef struct muon_plan_opts {
  uint32_t struct_size;         /* sizeof(muon_plan_opts); set by muon_plan_opts_default */
  int32_t nesterov;             /* 1 (default): d = g + beta*buf;  0: d = buf */
  float eps;                    /* added to ||d||_F before dividing; default 1e-7 */
  float rms_scale;              /* s = rms_scale * sqrt(max(rows, cols)); default 0.2 */
  int32_t precision;            /* muon_precision, default AUTO */
  int32_t form;                 /* muon_form, default AUTO */
  int32_t tile;                 /* tile plan of the bf16 NS kernels, -1 (default): chosen per
                                   shape; 0..9 force one plan for every bf16 matrix (the
                                   symmetric and the m x n products' output tiles:
                                   0: 128/128x128, 1: 128/256x256, 2: 256/256x256,
                                   3: 128/256x128, 4: 128/128x256; 5, 6, 7: plans 0, 1, 2
                                   with the m x n product reading X k-major, so no
                                   transposed copy of X is kept; 8: 64/256x256 and
                                   9: 64/128x128, both k-major).  Ignored on the fp32
                                   path */
  int32_t tune;                 /* muon_tune, default ONCE (OFF when no cache path is known) */
  int32_t host_only;            /* 1: plan on the host only - no device, no workspace, no
                                   timing; muon_step refuses such a plan (planner tests) */
  int32_t lanes;                /* concurrent NS lanes per chunk: the chunk's matrices are cut
                                   into this many runs of about equal work whose NS stages go
                                   to their own streams (forked from and joined back into the
                                   caller's stream).  0 (default): 1, or the count the
                                   whole-set timing picks when tuning; 1..4: forced */
  uint64_t workspace_cap_bytes; /* 0: default (96 GiB).  Matrices are processed in chunks
                                   whose workspace fits the cap; one matrix over it: ENOMEM */
  const char* cache_path;       /* tune cache file; NULL: $MUON_TUNE_CACHE, else no cache */
} muon_plan_opts;

typedef struct muon_plan muon_plan;

/* Summary of a plan (host memory, filled by muon_plan_info). */
typedef struct muon_plan_info {
  int32_t n_matrices;
  int32_t n_groups;           /* distinct (canonical shape, precision, form, tile) keys */
  int32_t n_chunks;           /* workspace chunks (1 unless the cap forces more) */
  int32_t n_gram;             /* matrices that run the Gram-space form */
  uint64_t workspace_bytes;   /* device workspace the plan owns */
  double ns_flops_min;        /* per step at the default T = 5: symmetric-aware algorithmic flops */
  double ns_flops_issued;     /* per step at T = 5: flops the chosen tiles actually issue */
  double ew_bytes;            /* per step: algorithmic HBM bytes of the elementwise kernels */
  uint64_t plan_hash;         /* FNV-1a of the canonical serialization */
  int32_t n_lanes;            /* concurrent NS lanes per chunk (muon_plan_opts.lanes) */
  int32_t reserved;
} muon_plan_info;

/* Per-kernel timing collected while profiling is on (see muon_plan_set_profiling):
 * one entry per (stage, kernel) pair. */
typedef struct muon_kernel_time {
  char name[32];        /* stage, e.g. "ns_apply", "ew_momentum" */
  char kernel[32];      /* kernel instance, e.g. "k_nt<256,256,bf16>" */
  int64_t launches;     /* launches timed */
  double total_ms;      /* summed dispatch time (hipEvent pairs) of those launches */
  double flops;         /* summed algorithmic flops of those launches (0 for elementwise) */
  double bytes;         /* summed algorithmic HBM bytes of those launches */
} muon_kernel_time;

/* One profiled launch: its dispatch start and end as times from the first
 * launch recorded since profiling was enabled or the totals were last reset. */
typedef struct muon_launch_interval {
  char name[32];        /* stage */
  char kernel[32];      /* kernel instance */
  double start_ms, end_ms;
} muon_launch_interval;

/* Fills *opts with the defaults listed above.  NULL: EINVAL. */
int muon_plan_opts_default(muon_plan_opts* opts);

/*
 * Builds a plan for n matrices (descs: host array of n).  Groups matrices by
 * canonical shape (m = min(rows, cols), n = max) and precision; picks per group
 * the NS form and tile plan (timed once and cached, or by the cost model); lays
 * the groups out in chunks under the workspace cap; allocates the device
 * workspace on the current HIP device (except host_only).  The plan owns its
 * workspace; release it with muon_plan_destroy.  Given the same descs, options
 * and cache contents the plan is byte-identical (muon_plan_serialize).
 * opts NULL: defaults.  Errors: EINVAL (NULL descs/out, n <= 0, reserved != 0,
 * an option out of range), EUNSUPPORTED (dtype; rows or cols < 1; the smaller
 * side over 16384, the larger over 2^20, or min * max (each rounded up to 256)
 * over 2^30; no gfx950 device), ENOMEM, EHIP.
 */
int muon_plan_create(const muon_matrix_desc* descs, int n, const muon_plan_opts* opts,
                     muon_plan** out);

/* Frees the plan and its workspace (waits for the device first).  NULL: no-op, OK. */
int muon_plan_destroy(muon_plan* plan);

/*
 * One Muon step over all matrices of the plan, enqueued on `stream`; returns
 * without waiting for the device.  params, grads, momenta: host arrays of n
 * device pointers in the order of the plan's descs (params and grads in the
 * matrix dtype, momenta fp32).  params and momenta are updated in place; grads
 * are read only.  coeffs: host pointer to (a, b, c) used at every NS step, or
 * NULL for (3.4445, -4.7750, 2.0315).  ns_steps = 0 applies the normalized
 * Nesterov direction.  The plan's workspace is shared by its calls: do not run
 * two steps of one plan concurrently on different streams.
 * Errors: EINVAL (NULL array or entry, ns_steps < 0 or > 64, non-finite scalar),
 * ESTATE (host-only plan; changed pointers on a stream under capture), EHIP
 * (launch failure).
 */
int muon_step(muon_plan* plan, void* const* params, const void* const* grads,
              float* const* momenta, float lr, float beta, float wd, int ns_steps,
              const float* coeffs, void* stream);

/* As muon_step with a per-step coefficient schedule: coeffs holds 3*ns_steps
 * floats, (a_k, b_k, c_k) for step k.  coeffs may be NULL only if ns_steps = 0. */
int muon_step_schedule(muon_plan* plan, void* const* params, const void* const* grads,
                       float* const* momenta, float lr, float beta, float wd, int ns_steps,
                       const float* coeffs, void* stream);

/*
 * Test hook: while set, every muon_step also writes the fp32 update
 * U = -lr * (wd * W + s * X_T) of matrix i, before rounding to the parameter
 * dtype, to dst[i] (device pointer, rows x cols fp32, row-major).  dst is a host
 * array of n device pointers (an entry may be NULL); dst = NULL turns it off.
 */
int muon_plan_set_update_capture(muon_plan* plan, float* const* dst);

/*
 * Non-finite detection: bit 0 of *flags is set when some matrix had a
 * non-finite ||d||_F in a step since the last clear (its X is then NaN and so
 * is its update).  Synchronizes the device.  clear != 0 resets the flag.
 */
int muon_plan_get_flags(muon_plan* plan, uint32_t* flags, int clear);

/*
 * Canonical plan bytes (groups, forms, tiles, chunks, launch order).  buf NULL:
 * *len receives the size.  Otherwise *len is the capacity of buf; too small: EINVAL.
 */
int muon_plan_serialize(const muon_plan* plan, void* buf, size_t* len);

/* Fills *info.  EINVAL on NULL. */
int muon_plan_info_get(const muon_plan* plan, muon_plan_info* info);

/*
 * Per-matrix decision: form (muon_form DIRECT or GRAM), tile plan (see
 * muon_plan_opts.tile; 0 on the fp32 path), group index, chunk index and NS
 * lane (0 .. n_lanes-1; lane 0 runs on the caller's stream) of matrix i.  Any
 * out pointer may be NULL.  EINVAL: NULL plan or i out of range.
 */
int muon_plan_matrix_choice(const muon_plan* plan, int i, int32_t* form, int32_t* tile,
                            int32_t* group, int32_t* chunk, int32_t* lane);

/*
 * Profiling: while enabled, muon_step (and muon_orthogonalize) record each
 * kernel's dispatch start and end in a hipEvent pair (hipExtLaunchKernel), and
 * run the NS lanes one after another on the step's stream, so every recorded
 * time is one kernel's alone (the events also hold the few microseconds of the
 * dispatch itself).  Timing with profiling off is therefore not comparable.
 * muon_plan_get_kernel_times synchronizes,
 * folds the recorded pairs into per-(stage, kernel) totals, sorted by stage then
 * kernel name, and writes up to max entries to out (host array), the count to
 * *n_out.  reset != 0 clears the totals (and the intervals) after.
 * muon_plan_get_launch_intervals writes, in launch order, up to max of the
 * launches folded so far (by muon_plan_get_kernel_times) to out and their
 * count to *n_out.
 */
int muon_plan_set_profiling(muon_plan* plan, int enable);
int muon_plan_get_kernel_times(muon_plan* plan, muon_kernel_time* out, int max, int* n_out,
                               int reset);
int muon_plan_get_launch_intervals(const muon_plan* plan, muon_launch_interval* out, int max,
                                   int* n_out);

/* Thread-local text of the last error on this thread ("" if none).  Never NULL. */
const char* muon_last_error(void);

/*
 * Newton-Schulz orthogonalization alone ("DeepSpeed now supports Muon"
 * (setupai.cc), technical deep dive: the orthogonalization Muon applies to
 * the update; here without momentum, scale or weight decay): for every matrix
 * i of the plan, out_i = NS_T(M_i / (||M_i||_F + eps)) with the plan's form,
 * tile plan and precision, in the stored orientation (a tall matrix is
 * iterated transposed and transposed back).
 *   inputs   host array of n device pointers, rows x cols row-major in the
 *            matrix's plan dtype; read only
 *   outputs  host array of n device pointers, rows x cols row-major fp32
 *   coeffs   host, 3*ns_steps floats (a_k, b_k, c_k), one triple per step;
 *            NULL: the quintic (3.4445, -4.7750, 2.0315) at every step
 * ns_steps = 0 gives the normalized input.  Asynchronous on stream; it uses
 * the plan's workspace, so it must not overlap a muon_step or another call on
 * the same plan.  A non-finite norm sets the flag muon_plan_get_flags reads.
 * EINVAL (NULL array or pointer, ns_steps outside [0, 64], non-finite
 * coefficient), ESTATE (host-only plan; changed pointers on a stream under
 * capture), EHIP (launch error).
 */
int muon_orthogonalize(muon_plan* plan, const void* const* inputs, float* const* outputs,
                       int ns_steps, const float* coeffs, void* stream);

/*
 * Estimated step time of matrix i in microseconds (*us): the NS time per
 * matrix that its shape measured when the plan was tuned (the cost model's
 * estimate otherwise) plus its elementwise bytes at 5 TB/s.  This is the cost
 * muon_assign_owners balances.  EINVAL: NULL plan or us, i out of range.
 */
int muon_plan_matrix_cost(const muon_plan* plan, int i, double* us);

/*
 * Owner assignment (DMuon announcement (wjxwpt.net), improvement 3
 * "computation-aware load balancing"): every item (matrix) goes to exactly
 * one of n_owners owners so that the largest per-owner total cost (the
 * makespan) is minimal.  Exact depth-first branch and bound seeded with the
 * LPT schedule (largest item first, to the least-loaded owner); when the
 * search exceeds node_limit nodes (<= 0: 2,000,000) the best schedule found is
 * improved by moves and swaps off the most loaded owner and returned as not
 * proven optimal.  Host-only: no device is used.
 *   costs      host array of n finite, non-negative costs (any unit)
 *   owner      host array of n, receives each item's owner in [0, n_owners)
 *   makespan   nullable; receives the schedule's makespan
 *   optimal    nullable; receives 1 if the makespan is proven minimal, else 0
 * EINVAL: n < 0, n_owners < 1, NULL costs or owner with n > 0, a negative or
 * non-finite cost.  Deterministic: equal inputs give equal assignments.
 */
int muon_assign_owners(const double* costs, int n, int n_owners, int64_t node_limit,
                       int32_t* owner, double* makespan, int32_t* optimal);

/*
 * Fused multi-tensor AdamW for the parameters that do not go to Muon
 * ("DeepSpeed now supports Muon" (setupai.cc), technical deep dive: the
 * usual hybrid runs Muon on the weight matrices and AdamW on embeddings,
 * biases and the final classifier).  The pages do not write AdamW out; this is
 * AdamW with decoupled weight decay as published (Loshchilov and Hutter), per
 * element, t = step >= 1:
 *   m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2
 *   p <- p (1 - lr wd) - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * in fp32 arithmetic; p stored back in its dtype (bf16: round to nearest even).
 * The hyperparameters are doubles: 1 - beta, the bias corrections and
 * 1 - lr wd are formed in double on the host before rounding to fp32.
 *
 * muon_adamw_plan_create: n tensors of numels[i] >= 1 elements with params and
 * grads of dtypes[i] (MUON_F32 or MUON_BF16); moments are fp32.  Needs a
 * current HIP device (gfx950); owns a small device table.  EINVAL (NULL, n <= 0),
 * EUNSUPPORTED (dtype, numel < 1), ENOMEM, EHIP.
 *
 * muon_adamw_step: host arrays of n caller-owned device pointers (contiguous,
 * numels[i] elements each); params, exp_avg and exp_avg_sq updated in place,
 * grads read only.  One launch on stream, asynchronous.  EINVAL (NULL pointer,
 * step < 1, beta outside [0, 1), eps < 0, non-finite lr, wd or eps), ESTATE
 * (changed pointers on a stream under capture), EHIP.
 */
typedef struct muon_adamw_plan muon_adamw_plan;
int muon_adamw_plan_create(const int64_t* numels, const int32_t* dtypes, int n,
                           muon_adamw_plan** out);
int muon_adamw_step(muon_adamw_plan* plan, void* const* params, const void* const* grads,
                    float* const* exp_avg, float* const* exp_avg_sq, double lr, double beta1,
                    double beta2, double eps, double wd, int64_t step, void* stream);
int muon_adamw_plan_destroy(muon_adamw_plan* plan);

/*
 * Graph replay of muon_step / muon_step_schedule (enable != 0), for callers
 * whose step is bound by launch overhead (few or small matrices) and whose
 * arguments repeat from step to step.  The first step with a given set of
 * arguments (the params, grads and momenta pointers, the update capture
 * buffers, lr, beta, wd, ns_steps and the coefficients) runs as usual; the
 * next step with the same arguments is captured into a HIP graph (stream
 * capture, thread-local mode) and launched; later steps with the same
 * arguments launch that graph again.  Any other argument set starts over
 * (eager, then a new capture); the tensors' contents may change freely.  With
 * lr or a coefficient changing every step, nothing is ever replayed.  The
 * graph holds kernel launches and the lanes' event dependencies only (no
 * memory set or copy nodes); a changed pointer table is uploaded before the
 * graph launches.  Needs a stream other than the null stream (EINVAL on
 * muon_step otherwise); profiling steps always run eagerly, and so do steps
 * enqueued while the caller is capturing the stream into a graph of its own
 * (the launches then go into the caller's graph).  enable = 0
 * waits for the device and releases the graph.  EINVAL (NULL plan), ESTATE
 * (host-only plan).
 */
int muon_plan_set_graph(muon_plan* plan, int enable);

/*
 * Ceiling probes (measurement only; not part of a step).  They give the rates
 * this part sustains when nothing else limits them, so a kernel's figure can be
 * read against a measured ceiling beside the published peak (dense bf16 MFMA
 * about 2.5 PFLOP/s, HBM3E 8 TB/s).  Both need a current HIP device, first
 * wait for all earlier work on it, run on a stream of their own (default
 * priority) and return when done: one warm-up launch, then the timed
 * launch(es) between two events.
 *
 * muon_probe_mfma_bf16: 2 blocks of 4 waves per compute unit; every wave runs
 * iters rounds of 4 independent v_mfma_f32_32x32x16_bf16 accumulations on
 * register operands (no memory traffic; 32768 flop each).  tflops receives
 * flop / time / 1e12, flops (nullable) the flop count of the timed launch.
 * Allocates and frees a small output buffer (one float per thread).
 * EINVAL: iters outside [1, 2^24], NULL tflops.  EHIP: device or launch error.
 *
 * muon_probe_hbm_copy: copies `bytes` from src to dst (caller-owned device
 * buffers, 16-byte aligned, non-overlapping; bytes a non-zero multiple of 16)
 * with 16-byte accesses, for each of eight launch variants (grid-stride over
 * 4, 8 or 16 blocks of 256 threads per compute unit, or one block per
 * contiguous 16 KiB run; plain or nontemporal loads and stores): one warm-up
 * copy, then reps timed copies.  gbs receives the
 * best variant's 2 * bytes * reps / time / 1e9 (read plus written bytes).  Use
 * buffers well above the 256 MB last-level cache to measure HBM.
 * EINVAL: NULL pointer, size or alignment, overlap, reps outside [1, 1000].
 * EHIP: launch error.
 */
int muon_probe_mfma_bf16(int iters, double* tflops, double* flops);
/* As muon_probe_mfma_bf16, but each MFMA of a round of eight takes another of
 * eight pairs of random bf16 register operands (random signs and mantissas):
 * the switching activity of real data.  The part is power-limited under dense
 * MFMA load, so this rate, not the fixed-operand one, is the ceiling a
 * contraction on random data is read against. */
int muon_probe_mfma_bf16_random(int iters, double* tflops, double* flops);
int muon_probe_hbm_copy(void* dst, const void* src, uint64_t bytes, int reps, double* gbs);
/* The NT contraction core of the large NS products (256x256 tiles of 8
 * waves, k-tiles of 64 copied global -> LDS, two stages) alone, without an
 * epilogue: one launch computes every 256x256 tile of P Q^T (P: m x k, Q:
 * n x k, bf16 row-major, caller-owned device buffers, 16-byte aligned; m and
 * n positive multiples of 256, k a positive multiple of 64, m k and n k below
 * 2^31) and keeps only each thread's sum of its accumulators.  One warm-up
 * launch, then reps timed launches; tflops receives 2 m n k reps / time /
 * 1e12; checksum (nullable) the sum over all tiles of their accumulator sums,
 * i.e. the sum of all entries of P Q^T as the kernel accumulated it.  Read a
 * kernel against this rate to see what its epilogue, tile order and operand
 * traffic cost beyond the core.  Allocates and frees a small output buffer.
 * EINVAL: NULL pointer, sizes, alignment, reps outside [1, 100].  EHIP:
 * device or launch error. */
int muon_probe_nt_bf16(const void* P, const void* Q, int m, int n, int k, int reps, double* tflops,
                       double* checksum);
/* The same core with an epilogue shaped as the NS products' bf16 one, to
 * read what writing the product costs: every 256x256 tile of P Q^T is
 * rounded to bf16 (nearest even), staged once in LDS and stored by a row
 * pass into C (m x n row-major); mode 2 adds a column pass storing the tile
 * transposed into CT (n x m row-major, the shape of a transposed copy or a
 * mirrored tile); mode 3 is mode 2 with nontemporal stores.  P, Q, C, CT:
 * caller-owned device buffers, 16-byte aligned (CT unused and nullable in
 * mode 1); sizes as muon_probe_nt_bf16, m n below 2^30.  One warm-up launch,
 * then reps timed launches; tflops receives 2 m n k reps / time / 1e12.
 * EINVAL: NULL pointer, mode, sizes, alignment, reps outside [1, 100].
 * EHIP: device or launch error. */
int muon_probe_nt_out_bf16(const void* P, const void* Q, void* C, void* CT, int m, int n, int k, int mode,
                           int reps, double* tflops);

/*
 * One Muon step of ONE matrix that allocates no device memory, for callers
 * that cannot call hipMalloc (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The same update as muon_step on
 * that matrix, with a fixed configuration instead of a plan: direct NS form,
 * 128 x 128 tiles for every product (on the bf16 path the m x n product reads
 * X k-major, as tile plan 5 does), no timing, no lanes.  The workspace, the
 * norm partials, the scale, the matrix descriptor and the work-item lists live
 * in one static device array of 64 MiB per device that the library holds
 * until the process ends; a call enqueues kernels only (a set-up kernel writes
 * the tables into that array), so it can be captured into a graph.
 *   desc      host; rows, cols >= 1, dtype MUON_F32 or MUON_BF16, reserved 0
 *   opts      host, nullable (defaults); nesterov, eps and rms_scale are used;
 *             form GRAM or precision other than AUTO: EUNSUPPORTED; the other
 *             fields are ignored
 *   param     device, rows x cols row-major in desc.dtype, updated in place
 *   grad      device, same shape and dtype, read only
 *   momentum  device, rows x cols fp32, updated in place
 *   coeffs    host, (a, b, c) used at every NS step; NULL: the quintic
 * Size limit: with m = min(rows, cols) and n = max(rows, cols) each rounded up
 * to 128, the workspace 4 (m n + m m) bytes (bf16) or 12 m n + 8 m m bytes
 * (fp32), plus under 0.3 MiB of tables, must fit 64 MiB (e.g. bf16 2048 x
 * 4096 or 1024 x 8192; fp32 1024 x 4096); larger: ENOMEM, nothing enqueued.
 * Every call on a device uses that device's one array and leaves its contents
 * there: calls that overlap on one device (different streams, unordered
 * threads) race; calls in order on one stream are safe.  No non-finite flag is
 * reported.  Errors: EINVAL (NULL pointer, ns_steps outside [0, 64],
 * non-finite scalar or coefficient, opts.struct_size), EUNSUPPORTED (dtype,
 * zero or over-large size, no gfx950 device, form / precision), ENOMEM (over
 * the array), EHIP (symbol lookup or launch error).
 */
int muon_step_noalloc(const muon_matrix_desc* desc, const muon_plan_opts* opts, void* param,
                      const void* grad, float* momentum, float lr, float beta, float wd,
                      int ns_steps, const float* coeffs, void* stream);

/* MUON_ABI_VERSION of the library. */
int muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
