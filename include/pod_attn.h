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

/* Scheduler modes of the fused kernel: how the two workgroups of each CU
 * pick their first role (every workgroup moves to the other queue when its
 * own runs dry, so all modes run every unit exactly once). */
typedef enum {
  /* The planner's choice (currently POD_SCHED_SPLIT). */
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

typedef struct pod_attn_plan_s* pod_attn_plan_t;   /* opaque, library-owned */

typedef struct {
  int32_t num_qo_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* must be 128 */
  int32_t kv_layout;      /* pod_kv_layout_t */
  int32_t page_size;      /* PAGED: power of two in [1, 1024]; ignored otherwise */
  int32_t causal;         /* 1: bottom-right causal chunks; 0: full visibility */
  float sm_scale;         /* finite, > 0; multiplies the fp32 score */
} pod_attn_params_t;

typedef struct {
  int32_t wgs_per_cu;            /* 0 = auto; only 2 is supported (one
                                    prefill-capable wave per SIMD pair) */
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
  int32_t num_partials;
  int32_t trace_records;
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
 *   k, v       device bf16 CONTIGUOUS: [sum(kv_len), Hkv, 128] with request r's
 *                          tokens at rows kv_indptr[r] ..;
 *                          PAGED: [num_pages, page_size, Hkv, 128]; token t of
 *                          request r is slot t % page_size of page
 *                          page_indices[page_indptr[r] + t / page_size]
 *   kv_indptr    device int32 [num_prefill + num_decode + 1]  (CONTIGUOUS)
 *   page_indptr  device int32 [num_prefill + num_decode + 1]  (PAGED)
 *   page_indices device int32 [page_indptr[last]]             (PAGED)
 *   o_prefill, o_decode     device bf16, shapes of q_prefill / q_decode
 *   lse_prefill, lse_decode device fp32 [rows, Hq], natural log; may be NULL
 * Request order everywhere: the prefill requests, then the decodes.  Slots of
 * pages past a request's kv_len are never read.  Base pointers must be 16-byte
 * aligned. */
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
} pod_attn_tensors_t;

/* Plans one hybrid batch for the current HIP device.
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
 * Errors: POD_ERR_INVALID_ARGUMENT (lengths, heads, scale, layout, NULL
 * length arrays with a nonzero count), POD_ERR_UNSUPPORTED (head_dim != 128,
 * wgs_per_cu other than 0 or 2), POD_ERR_WORKSPACE_TOO_SMALL, POD_ERR_HIP. */
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

/* Fused run: one persistent kernel (two workgroups per CU) for all prefill
 * tiles and decode splits, then the merge kernel if any split exists.
 * Asynchronous on `stream`.
 * Errors: POD_ERR_INVALID_ARGUMENT (NULL plan/tensors, a required pointer
 * NULL or not 16-byte aligned, plan without workspace), POD_ERR_HIP. */
pod_status_t pod_attn_run(pod_attn_plan_t plan, const pod_attn_tensors_t* t,
                          hipStream_t stream);

/* pod_attn_run that also records two caller-created events on `stream`,
 * immediately before and after the fused kernel's launch (the merge kernel,
 * when any, follows `after_fused`), so that the fused kernel alone can be
 * timed.  Either event may be NULL (not recorded).  The work done is exactly
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

/* Counts of a plan.  Errors: POD_ERR_INVALID_ARGUMENT on NULL. */
pod_status_t pod_attn_plan_info(pod_attn_plan_t plan, pod_attn_plan_info_t* out);

/* Copies one of the plan's host work lists into dst (host int32, capacity n
 * elements); *count receives the element count (dst may be NULL to query).
 * which: 0 fused prefill items (8 int32 each), 1 fused decode items (8 each),
 * 2 fused merge tasks (4 each), 3/4/5 the sequential lists, 6/7 the fused /
 * sequential prefill pool offsets (num_xcds + 1 each).  Item fields are
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

#ifdef __cplusplus
}
#endif
#endif /* POD_ATTN_H_ */
