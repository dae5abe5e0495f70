/*
 * pod_attn.h - C ABI of libpod_attn.so: fused prefill+decode attention of one
 * hybrid batch on an AMD MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [POD] "POD-Attention: Unlocking Full Prefill-Decode Overlap for Faster LLM
 *         Inference" (ASPLOS 2025), summary page.
 *   [PR]  "Limit kv split when prefill tokens <= 1536" (pull request #1 of a
 *         FlashInfer fork, H200 benchmark log).
 *   [PAT] "PAT: Accelerating LLM Decoding via Prefix-Aware Attention with
 *         Resource Efficient Multi-Tile Kernel" (catalogue record, abstract).
 *
 * The operation ([POD] "Why this problem is worth solving"; "The argument in
 * one glance"): a hybrid batch holds prefill requests (a chunk of qo_len new
 * tokens at the end of a kv_len-token context, causal) and decode requests
 * (one new token looking at its whole kv_len-token KV cache).  For request r,
 * query head h and chunk row i (absolute position p = kv_len - qo_len + i):
 *
 *     s_j  = sm_scale * <q[i,h,:], k[j, h / (Hq/Hkv), :]>   for visible j
 *     O[i,h,:] = sum_j softmax(s)_j * v[j, h / (Hq/Hkv), :]
 *     LSE[i,h] = ln sum_j exp(s_j)
 *
 * with visible j = 0..p when causal (bottom-right alignment), else all keys.
 * A decode token is the qo_len = 1 case.  The pages give no formula or layout;
 * these readings are the library's contract.
 *
 * pod_attn_run executes both parts in ONE kernel launch whose workgroups pick
 * their role (prefill tile or decode split) at run time from a per-CU counter
 * ([POD] "How POD-Attention overlaps" > "Fuse prefill and decode attention
 * into one kernel", "Self-assign roles per SM in software"), followed by a
 * log-sum-exp merge of KV-split partials when the plan splits ([POD] "Cap
 * prefill splitting to avoid contention"; [PAT] abstract, final merge).
 * pod_attn_sequential_run is the baseline the pages compare against: the
 * prefill kernel, then the decode kernel, then the merge, on one stream
 * ([POD] "What people did before": separate kernels run back to back).
 *
 * Conventions for every function:
 *   - returns pod_status_t; never throws, aborts or prints;
 *   - on a non-OK status, pod_attn_last_error() returns a thread-local text;
 *   - "host" pointers are read during the call only; "device" pointers must
 *     stay valid until the work enqueued on the stream has finished.
 */
#ifndef POD_ATTN_H_
#define POD_ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POD_OK = 0,
  POD_ERR_INVALID_ARGUMENT = 1,   /* bad length, head count, scale, pointer */
  POD_ERR_UNSUPPORTED = 2,        /* valid request the library does not handle */
  POD_ERR_WORKSPACE_TOO_SMALL = 3,
  POD_ERR_HIP = 4,                /* a HIP runtime call failed (text says which) */
  POD_ERR_INTERNAL = 5
} pod_status_t;

typedef enum { POD_KV_CONTIGUOUS = 0, POD_KV_PAGED = 1 } pod_kv_layout_t;

/* Element type of the KV cache.  POD_KV_FP8_E4M3: OCP FP8 E4M3 bytes with
 * one fp32 scale per KV head for K and one for V (value = decoded byte times
 * its head's scale); a lever on decode's bytes named in "Prefill vs. Decode
 * GPU Utilization Imbalance", section "Quantization and compression as a
 * lever on both the bandwidth and capacity problem".  Supported for every
 * batch (prefill, decode or both) with a contiguous cache or pages of >= 16
 * tokens; the prefill tile converts each staged K/V tile to 16-bit in LDS
 * (K to bf16, V to fp16) and runs its PV product on fp16 P, the decode unit
 * converts in registers. */
typedef enum { POD_KV_BF16 = 0, POD_KV_FP8_E4M3 = 1 } pod_kv_dtype_t;

/* Scheduler modes of the fused kernel: how the two workgroups of each CU
 * pick their first role (every workgroup moves to the other queue when its
 * own runs dry, so all modes run every unit exactly once). */
typedef enum {
  /* The planner's choice: for a batch of at most two fused units (prefill
   * items + decode groups) per workgroup slot, one workgroup per unit
   * (POD_FLAG_ONE_UNIT_PER_WG) with POD_SCHED_COLOCATE roles when the batch
   * has one prefill request and POD_SCHED_SPLIT roles when it has several;
   * otherwise POD_SCHED_SPLIT with persistent workgroups. */
  POD_SCHED_AUTO = 0,
  /* Co-location on every CU: the CU's workgroups take roles in arrival
   * order (a per-CU ticket), the first prefill_quarters_per_cu / 4 of them
   * (in quarters, spread over neighbouring CUs) prefill, the rest decode
   * ([POD] "Self-assign roles per SM in software"). */
  POD_SCHED_COLOCATE = 1,
  /* No role steering: every workgroup takes prefill units while they last,
   * then decode units (a fused launch without co-location control). */
  POD_SCHED_ORDERED = 2,
  /* CU-level partition: every workgroup of a CU takes the same first role;
   * prefill_quarters_per_cu / 8 of the CUs start on prefill tiles, the rest
   * on decode units.  On MI355X one wave per SIMD cannot keep the matrix
   * cores busy, so prefill runs best two waves per SIMD on fewer CUs while
   * decode saturates HBM from the others. */
  POD_SCHED_SPLIT = 3
} pod_sched_mode_t;

/* tuning flags */
#define POD_FLAG_TRACE 0x1u   /* fused run (and, with match_sequential, sequential
                                 run) records one pod_trace_record_t per unit */
#define POD_FLAG_BATCHED_PREFILL 0x2u  /* the plan also builds (and its workspace
                                 holds) the work list of pod_attn_batched_prefill_run */
#define POD_FLAG_ONE_UNIT_PER_WG 0x4u  /* fused launch of one workgroup per unit
                                 (prefill items + decode groups) instead of two
                                 persistent workgroups per CU: each takes its role
                                 as the scheduler mode says, runs one unit of it (or
                                 of the other role when its own is exhausted) and
                                 exits, the hardware refilling the slot -- the
                                 launch shape of [POD] "Fuse prefill and decode
                                 attention into one kernel" */

typedef struct pod_attn_plan_s* pod_attn_plan_t;   /* opaque, library-owned */

typedef struct {
  int32_t num_qo_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* must be 128 */
  int32_t kv_layout;      /* pod_kv_layout_t */
  int32_t page_size;      /* PAGED: power of two in [1, 1024]; ignored otherwise */
  int32_t causal;         /* 1: bottom-right causal chunks; 0: full visibility */
  float sm_scale;         /* finite, > 0; multiplies the fp32 score */
  int32_t kv_dtype;       /* pod_kv_dtype_t */
} pod_attn_params_t;

typedef struct {
  int32_t wgs_per_cu;            /* 0 = auto; only 2 is supported.  The pages
                                    run 2 or 4 blocks per SM ([POD] "How
                                    POD-Attention overlaps" > "Balance shared
                                    memory and threadblock count"); here a
                                    prefill workgroup needs 64 KiB of LDS and
                                    256 VGPRs per lane, so only two fit a CU
                                    (4 returns POD_ERR_UNSUPPORTED) */
  int32_t prefill_quarters_per_cu; /* prefill share q in 0..4*wgs_per_cu
                                    (eighths of the workgroup slots); -1 =
                                    auto (proportional to the estimated
                                    prefill and decode times, [POD] "The
                                    idea").  SPLIT: the CUs whose index in
                                    their shader array is below q start on
                                    prefill; COLOCATE: the first q/4 of each
                                    CU's workgroups do */
  int32_t prefill_kv_splits;     /* 0 = auto; >0 forces this many KV splits per
                                    prefill tile (capped by its 64-key tiles and
                                    by 64) */
  int32_t decode_kv_splits;      /* 0 = auto; >0 forces this many KV splits per
                                    decode request (capped by its 32-key steps and
                                    by 64) */
  int32_t match_sequential;      /* 1: sequential_run uses the fused plan's work
                                    lists (for bitwise comparisons) */
  int32_t sched_mode;            /* pod_sched_mode_t */
  uint32_t flags;                /* POD_FLAG_* */
} pod_attn_tuning_t;

/* Device shape the planner targets.  pod_attn_plan queries the current device;
 * pod_attn_plan_host takes it from the caller (no GPU needed). */
typedef struct {
  int32_t num_cus;        /* compute units (MI355X: 256) */
  int32_t num_xcds;       /* accelerator dies with their own L2 (MI355X: 8) */
} pod_device_desc_t;

/* Counts describing a plan (pod_attn_plan_info). */
typedef struct {
  int32_t prefill_items, decode_items, decode_groups, merge_tasks;
  int32_t seq_prefill_items, seq_decode_items, seq_merge_tasks;
  int32_t prefill_splits_max, decode_splits_max;
  int32_t wgs_per_cu, prefill_quarters_per_cu, sched_mode;
  int32_t one_unit_per_wg;     /* 1: the fused launch runs one workgroup per unit */
  int32_t num_partials;
  int32_t trace_records;
  int32_t runs_sequential;     /* 1: pod_attn_run runs the prefill and decode
                                  kernels back to back; 2: at once, on the
                                  caller's stream and the library's second
                                  stream on the device (see pod_attn_run) */
  uint64_t workspace_bytes;
} pod_attn_plan_info_t;

/* One unit of a fused run (POD_FLAG_TRACE): records 0 .. prefill_items-1
 * are the prefill items, then one per decode item. */
typedef struct {
  int32_t block;       /* blockIdx.x of the workgroup that ran it */
  int32_t cu_slot;     /* (xcc << 8) | (se << 5) | (sh << 4) | cu */
  int32_t role;        /* 0 prefill, 1 decode */
  int32_t unit;        /* prefill item or decode item index */
  uint64_t t_start;    /* s_memrealtime (100 MHz) when the unit started */
  uint64_t t_end;      /* s_memrealtime after the unit */
} pod_trace_record_t;

/* Tensors of one run.  bf16 = IEEE bfloat16.  Row-major, no padding:
 *   q_prefill  device bf16 [sum(prefill qo_len), Hq, 128]  (requests in order)
 *   q_decode   device bf16 [num_decode, Hq, 128]
 *   k, v       device bf16 (or E4M3 bytes, kv_dtype FP8) CONTIGUOUS:
 *                          [sum(kv_len), Hkv, 128] with request r's
 *                          tokens at rows kv_indptr[r] ..;
 *                          PAGED: [num_pages, page_size, Hkv, 128]; token t of
 *                          request r is slot t % page_size of page
 *                          page_indices[page_indptr[r] + t / page_size]
 *   kv_indptr    device int32 [num_prefill + num_decode + 1]  (CONTIGUOUS)
 *   page_indptr  device int32 [num_prefill + num_decode + 1]  (PAGED)
 *   page_indices device int32 [page_indptr[last]]             (PAGED)
 *   o_prefill, o_decode     device bf16, shapes of q_prefill / q_decode
 *   lse_prefill, lse_decode device fp32 [rows, Hq], natural log; may be NULL
 *   k_scale, v_scale        device fp32 [Hkv] (kv_dtype FP8 only; else unused)
 * Request order everywhere: the prefill requests, then the decodes.  Slots of
 * pages past a request's kv_len are never read.  Base pointers must be 16-byte
 * aligned.  Unlike common paged-attention interfaces there is no per-request
 * last_page_len array: each request's kv_len is fixed when the plan is made
 * (the work lists are built from it), and the run reads no length from these
 * tensors. */
typedef struct {
  const void* q_prefill;
  const void* q_decode;
  const void* k;
  const void* v;
  const int32_t* kv_indptr;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  void* o_prefill;
  void* o_decode;
  float* lse_prefill;
  float* lse_decode;
  const float* k_scale;
  const float* v_scale;
} pod_attn_tensors_t;

/* Plans one hybrid batch for the current HIP device: validates the lengths,
 * builds the prefill tiles and decode units with their KV splits, and picks
 * the prefill:decode share of the GPU in proportion to the estimated prefill
 * and decode times ([POD] "The idea": proportional rather than even
 * allocation; "How POD-Attention overlaps" > "Cap prefill splitting to avoid
 * contention"; [PR] description: with at most 1536 prefill tokens the split
 * count is sized for the slots left beside the co-located decode work).
 *   prefill_qo_len/prefill_kv_len: host int32 [num_prefill], 1 <= qo <= kv
 *   decode_kv_len: host int32 [num_decode], >= 1
 *   tuning: host, may be NULL (all automatic)
 *   workspace: device buffer owned by the caller, or NULL to only query.
 * With workspace == NULL the call writes *workspace_needed and returns POD_OK
 * without creating a plan (*out_plan = NULL).  Otherwise it builds the plan,
 * enqueues the upload of its work lists and the zeroing of its counters on
 * `stream`, and returns a plan that refers to `workspace` (which must then
 * stay alive and unshared until pod_attn_plan_destroy).  Runs of one plan on
 * different streams must not overlap: they share the workspace.
 * Errors: POD_ERR_INVALID_ARGUMENT (lengths, heads, scale, layout, dtype,
 * NULL length arrays with a nonzero count), POD_ERR_UNSUPPORTED (head_dim !=
 * 128, wgs_per_cu other than 0 or 2, an FP8 cache with pages of fewer than
 * 16 tokens, or with the batched-prefill comparator, a kv_len above 2^24,
 * more than 2^31 - 1 (row, head) outputs, or KV splits whose partials
 * would number more than 2^31 - 1),
 * POD_ERR_WORKSPACE_TOO_SMALL, POD_ERR_HIP.  With an FP8 cache every run
 * entry point runs the FP8 forms of its kernels (fused: the FP8 prefill tile
 * beside the FP8 decode unit). */
pod_status_t pod_attn_plan(const pod_attn_params_t* params,
                           int32_t num_prefill, const int32_t* prefill_qo_len,
                           const int32_t* prefill_kv_len,
                           int32_t num_decode, const int32_t* decode_kv_len,
                           const pod_attn_tuning_t* tuning,
                           void* workspace, size_t workspace_bytes,
                           size_t* workspace_needed,
                           hipStream_t stream, pod_attn_plan_t* out_plan);

/* Same planning for an explicit device shape, with no HIP call at all; the
 * plan has no workspace and cannot run (host-side inspection and tests). */
pod_status_t pod_attn_plan_host(const pod_attn_params_t* params,
                                int32_t num_prefill, const int32_t* prefill_qo_len,
                                const int32_t* prefill_kv_len,
                                int32_t num_decode, const int32_t* decode_kv_len,
                                const pod_attn_tuning_t* tuning,
                                const pod_device_desc_t* device,
                                pod_attn_plan_t* out_plan);

/* Plans a decode-only batch whose requests share KV prefixes, the
 * pack-forward-merge of [PAT] (abstract: queries packed by shared prefix so
 * that the prefix's KV is loaded once; KV splitting; a final online-softmax
 * merge).
 *   decode_kv_len: host int32 [num_decode] (>= 1)
 *   prefix_group:  host int32 [num_decode]: the request's group in
 *                  [0, num_groups), or -1 (no shared prefix)
 *   prefix_len:    host int32 [num_groups]: tokens every member of the group
 *                  shares -- a whole number of pages, >= 1, no longer than any
 *                  member's kv_len.  The members' page tables must hold the
 *                  same pages for these tokens (the kernel reads the prefix
 *                  through the group's first member's table).
 * For each KV head, the rows of up to 64 / min(Hq/Hkv, 16) members are packed
 * into one workgroup tile over the prefix (four 16-row MFMA tiles sharing
 * every K/V step through LDS, so the prefix is read once per tile); each
 * member's own keys run as ordinary decode units; every (request, head)
 * result is merged by log-sum-exp.  pod_attn_plan_export lists the prefix
 * tiles as list 0 (in decode-item fields, up to 64 rows) and the suffix
 * units as list 1.  The trace and one-workgroup-per-unit flags are ignored
 * (the packed kernel has one launch shape and records no trace).
 * pod_attn_run runs this packed path; pod_attn_sequential_run and
 * pod_attn_streams_run run the ordinary (unshared) decode of the same batch,
 * the baseline.  Workspace, ownership and errors as pod_attn_plan, plus
 * POD_ERR_UNSUPPORTED for a contiguous or FP8 cache or the batched-prefill
 * flag, and POD_ERR_INVALID_ARGUMENT for group ids or prefix lengths out of
 * range. */
pod_status_t pod_attn_plan_shared_prefix(const pod_attn_params_t* params, int32_t num_decode,
                                         const int32_t* decode_kv_len,
                                         const int32_t* prefix_group, int32_t num_groups,
                                         const int32_t* prefix_len,
                                         const pod_attn_tuning_t* tuning, void* workspace,
                                         size_t workspace_bytes, size_t* workspace_needed,
                                         hipStream_t stream, pod_attn_plan_t* out_plan);

/* pod_attn_plan_shared_prefix without a GPU (host inspection, as
 * pod_attn_plan_host); the plan cannot run. */
pod_status_t pod_attn_plan_shared_prefix_host(const pod_attn_params_t* params,
                                              int32_t num_decode, const int32_t* decode_kv_len,
                                              const int32_t* prefix_group, int32_t num_groups,
                                              const int32_t* prefix_len,
                                              const pod_attn_tuning_t* tuning,
                                              const pod_device_desc_t* device,
                                              pod_attn_plan_t* out_plan);

/* pod_attn_plan for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the plan's workspace is a static 128 MiB device array of the library, one
 * per device, held until the process ends; the caller passes no workspace.
 * Arguments, validation and the returned plan are those of pod_attn_plan
 * (runs use it with pod_attn_run / pod_attn_sequential_run / ... as usual).
 * Allocates no device memory (no hipMalloc, hipFree or allocating library
 * routine; the plan object itself is host memory, freed by
 * pod_attn_plan_destroy) and creates no stream: a batch that pod_attn_plan
 * would run on two streams runs as one fused launch here.  The scratch is shared by every such plan on the
 * device: a new pod_attn_plan_scratch call overwrites the work lists and
 * counters of the previous one, so only the most recent scratch plan of a
 * device may run, and runs that overlap in time race.  The counters are
 * zeroed on `stream` by each call.
 * Errors: those of pod_attn_plan; POD_ERR_WORKSPACE_TOO_SMALL (with the
 * needed size) when the plan needs more than 128 MiB; POD_ERR_HIP when the
 * scratch address cannot be obtained. */
pod_status_t pod_attn_plan_scratch(const pod_attn_params_t* params,
                                   int32_t num_prefill, const int32_t* prefill_qo_len,
                                   const int32_t* prefill_kv_len,
                                   int32_t num_decode, const int32_t* decode_kv_len,
                                   const pod_attn_tuning_t* tuning, hipStream_t stream,
                                   pod_attn_plan_t* out_plan);

/* Fused run: one kernel for all prefill tiles and decode splits ([POD] "How
 * POD-Attention overlaps": prefill and decode in one launch, roles taken per
 * CU in software) -- persistent, two workgroups per CU, or one workgroup per
 * unit as the plan chose -- then the merge kernel if any split exists.  A
 * batch of one kind (no decodes, or no prefill; bf16 or FP8) has nothing to
 * overlap and runs the one kernel it needs with the sequential plan's lists,
 * i.e. what pod_attn_sequential_run runs (unless the plan traces: the trace
 * is indexed by the fused launch's units).  So does, under automatic
 * scheduling, an MHA batch (Hq == Hkv) too large for the one-unit launch
 * whose prefill is under a fifth of the planner's work estimate: its prefill items each stream their own KV head
 * and contend with the decode for HBM, and the fused launch measured slower
 * there.  A GQA batch (Hq > Hkv) with several prefill requests, too large
 * for the one-unit launch, whose prefill is under 0.15 of the estimate runs
 * the two kernels at once, the prefill kernel on `stream` and the decode
 * kernel on a second stream, forked from and joined back to `stream` by
 * events, as pod_attn_streams_run does (the library creates that stream, at
 * default priority, when the first such plan is made on a device, and keeps
 * it until the process ends; plans on the device share it): each kernel keeps its own
 * register and LDS footprint, which measured faster than the fused launch on
 * such decode-heavy batches (pod_attn_plan_info_t.runs_sequential reports the
 * choice; any explicit sched_mode keeps the fused launch).  A shared-prefix plan runs its
 * packed decode kernel.  Asynchronous on `stream`.
 * Errors: POD_ERR_INVALID_ARGUMENT (NULL plan/tensors, a required pointer
 * NULL or not 16-byte aligned, plan without workspace), POD_ERR_HIP. */
pod_status_t pod_attn_run(pod_attn_plan_t plan, const pod_attn_tensors_t* t,
                          hipStream_t stream);

/* pod_attn_run that also records two caller-created events on `stream`,
 * immediately before and after the fused kernel's launch (the merge kernel,
 * when any, follows `after_fused`), so that the fused kernel alone can be
 * timed; for a batch of one kind, around that one kernel.  Either event may be NULL (not recorded).  The work done is exactly
 * that of pod_attn_run.  Errors as pod_attn_run, plus POD_ERR_HIP when an
 * event cannot be recorded. */
pod_status_t pod_attn_run_events(pod_attn_plan_t plan, const pod_attn_tensors_t* t,
                                 hipStream_t stream, hipEvent_t before_fused,
                                 hipEvent_t after_fused);

/* Sequential baseline: prefill kernel, then decode kernel, then merge, on
 * `stream`.  Uses its own work lists (splits sized for a GPU running one
 * part at a time) unless the plan was made with match_sequential = 1.
 * Errors as pod_attn_run. */
pod_status_t pod_attn_sequential_run(pod_attn_plan_t plan, const pod_attn_tensors_t* t,
                                     hipStream_t stream);

/* Comparator of the pages: the sequential baseline's prefill kernel and
 * decode kernel launched on two streams so that the hardware may run them
 * concurrently ([POD] "What people did before, and where it broke": separate
 * kernels on concurrent streams give no control over co-location), then the
 * merge.  `decode_stream` (a different stream of default priority) first
 * waits for the work already enqueued on `stream`; the prefill kernel and the
 * merge run on `stream`, which waits for the decode kernel before the merge,
 * so work enqueued on `stream` afterwards sees the whole result.  Uses the
 * sequential plan's work lists.  Errors as pod_attn_run, plus
 * POD_ERR_INVALID_ARGUMENT when both streams are the same. */
pod_status_t pod_attn_streams_run(pod_attn_plan_t plan, const pod_attn_tensors_t* t,
                                  hipStream_t stream, hipStream_t decode_stream);

/* Comparator of the pages ("Batched Prefill" in the [PR] benchmark log): every
 * request of the batch goes through the prefill kernel in one launch, each
 * decode as a one-row chunk (a tile of its packed query heads at position
 * kv_len - 1), followed by the merge.  The plan must have been made with
 * POD_FLAG_BATCHED_PREFILL.  Errors as pod_attn_run, plus
 * POD_ERR_INVALID_ARGUMENT for a plan without that flag. */
pod_status_t pod_attn_batched_prefill_run(pod_attn_plan_t plan, const pod_attn_tensors_t* t,
                                          hipStream_t stream);

/* Log-sum-exp merge of KV-split partials ([PAT] abstract: the final merge of
 * per-split results by online softmax; [POD] "Cap prefill splitting to avoid
 * contention": attention split along the KV dimension).  For each row r:
 *     M = max_s lse_s,  L = M + ln sum_s exp(lse_s - M),
 *     O = sum_s exp(lse_s - L) * o_s
 * where partials with lse_s = -inf weigh nothing; a row whose partials are
 * all -inf gives O = 0 and L = -inf.
 *   part_o   device fp32 [n_rows, n_splits, 128], each partial normalised
 *            by its own softmax sum (16-byte aligned)
 *   part_lse device fp32 [n_rows, n_splits], natural log
 *   o        device bf16 [n_rows, 128] (16-byte aligned), written
 *   lse      device fp32 [n_rows], natural log, written; may be NULL
 * n_splits in [1, 64]; n_rows = 0 enqueues nothing.  Asynchronous on
 * `stream`.  Errors: POD_ERR_INVALID_ARGUMENT (counts, NULL or misaligned
 * pointers), POD_ERR_UNSUPPORTED (n_rows * n_splits >= 2^31), POD_ERR_HIP. */
pod_status_t pod_attn_merge(const float* part_o, const float* part_lse, int32_t n_rows,
                            int32_t n_splits, void* o, float* lse, hipStream_t stream);

/* Counts of a plan.  Errors: POD_ERR_INVALID_ARGUMENT on NULL. */
pod_status_t pod_attn_plan_info(pod_attn_plan_t plan, pod_attn_plan_info_t* out);

/* Copies one of the plan's host work lists into dst (host int32, capacity n
 * elements); *count receives the element count (dst may be NULL to query).
 * which: 0 fused prefill items (8 int32 each), 1 fused decode items (8 each),
 * 2 fused merge tasks (4 each), 3/4/5 the sequential lists, 6/7 the fused /
 * sequential prefill pool offsets (num_xcds + 1 each), 8/9/10 the
 * batched-prefill items, merge tasks and pool offsets, 11 the group members
 * of a shared-prefix plan (decode indices).  Item fields are
 * documented in plan.h of the sources.  Errors: POD_ERR_INVALID_ARGUMENT. */
pod_status_t pod_attn_plan_export(pod_attn_plan_t plan, int32_t which,
                                  int32_t* dst, size_t n, size_t* count);

/* Copies the trace of the last fused run (POD_FLAG_TRACE plans) to host
 * memory: up to n records; *count receives the number of records.
 * Synchronises `stream`.  Errors: INVALID_ARGUMENT, HIP. */
pod_status_t pod_attn_read_trace(pod_attn_plan_t plan, pod_trace_record_t* dst,
                                 size_t n, size_t* count, hipStream_t stream);

/* Frees the host plan object (not the caller's workspace).  NULL is a no-op. */
void pod_attn_plan_destroy(pod_attn_plan_t plan);

/* Thread-local description of the last non-OK status on this thread. */
const char* pod_attn_last_error(void);

/* Hardware-placement probe: launches `num_blocks` workgroups of 256 threads
 * that each write (hw_id register, xcc_id register) into out (device int32
 * [2 * num_blocks]).  Used to check the per-CU slot map on a device. */
pod_status_t pod_attn_probe_hwid(int32_t num_blocks, int32_t* out, hipStream_t stream);

/* HBM read-rate probe (measurement aid, not part of attention): launches
 * `num_blocks` workgroups of 256 threads that read bytes / 16 16-byte words
 * of `buf` (device, 16-byte aligned) once each with non-temporal loads and
 * write nothing, except to `sink` (device uint32) in the unlikely case that
 * the folded data equals a fixed constant.  Timing it with events on
 * `stream` gives the device's attainable read rate beside the datasheet
 * peak.  Errors: POD_ERR_INVALID_ARGUMENT, POD_ERR_HIP. */
pod_status_t pod_attn_probe_read_bw(const void* buf, size_t bytes, uint32_t* sink,
                                    int32_t num_blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* POD_ATTN_H_ */
