// C ABI of libpod_attn.so (declared in include/pod_attn.h).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/pod_attn.h"
#include "kernel_args.h"
#include "plan.h"

using namespace pod;

namespace {

thread_local std::string g_err;

pod_status_t set_err(pod_status_t st, const std::string& msg) {
  g_err = msg;
  return st;
}

pod_status_t hip_err(hipError_t e, const char* what) {
  return set_err(POD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

struct DevLists {              // byte offsets of one list set in the workspace
  size_t p_items = 0, d_items = 0, m_tasks = 0;
};

}  // namespace

struct pod_attn_plan_s {
  Batch batch;
  pod_attn_tuning_t tuning{};
  pod_device_desc_t dev{};
  PlanChoice choice;
  WorkLists fused, seq;
  bool seq_is_fused = false;
  int32_t n_partials = 0;
  int32_t trace_records = 0;
  // workspace layout (bytes)
  size_t off_counters = 0, off_trace = 0, off_part_lse = 0, off_part_o = 0;
  DevLists dl_fused, dl_seq;
  uint64_t launches[2] = {0, 0};   // successful launches per kind (counter parity)
  size_t ws_bytes = 0;
  char* ws = nullptr;          // caller-owned device buffer (NULL: host-only plan)
  int device = -1;
};

namespace {

pod_status_t build_plan(const pod_attn_params_t* params, int32_t np, const int32_t* qo,
                        const int32_t* pkv, int32_t nd, const int32_t* dkv,
                        const pod_attn_tuning_t* tuning, const pod_device_desc_t& dev,
                        pod_attn_plan_s* pl) {
  std::string err;
  pod_status_t st = validate(params, np, qo, pkv, nd, dkv, tuning, &err);
  if (st != POD_OK) return set_err(st, err);
  if (dev.num_cus < 1 || dev.num_xcds < 1 || dev.num_xcds > kMaxPools)
    return set_err(POD_ERR_INVALID_ARGUMENT, "device description out of range");
  pod_attn_tuning_t t{};
  t.prefill_quarters_per_cu = -1;
  if (tuning) t = *tuning;
  pl->tuning = t;
  pl->dev = dev;
  pl->batch.params = *params;
  pl->batch.qo.assign(qo, qo + np);
  pl->batch.pkv.assign(pkv, pkv + np);
  pl->batch.dkv.assign(dkv, dkv + nd);
  PlanChoice& c = pl->choice;
  c.wgs_per_cu = 2;
  c.sched_mode = t.sched_mode == POD_SCHED_AUTO ? POD_SCHED_SPLIT : t.sched_mode;
  c.prefill_quarters = t.prefill_quarters_per_cu >= 0
                           ? std::min(t.prefill_quarters_per_cu, 4 * c.wgs_per_cu)
                           : auto_prefill_quarters(pl->batch, c.wgs_per_cu, c.sched_mode);
  int64_t sum_qo = 0;
  for (int32_t x : pl->batch.qo) sum_qo += x;
  // Fused plan.  [PR]: with <= 1536 prefill tokens the prefill split count is
  // sized for the slots left beside the co-located decode workgroups (and
  // fewer items per slot); otherwise for every slot.
  const int64_t slots = (int64_t)dev.num_cus * c.wgs_per_cu;
  const int64_t p_slots_coloc = std::max<int64_t>(1, (int64_t)dev.num_cus * c.prefill_quarters / 4);
  const bool small_prefill = sum_qo <= 1536;
  const int64_t fused_p_slots = small_prefill ? p_slots_coloc : slots;
  const int64_t fused_d_waves =
      std::max<int64_t>(kWavesPerWG, (int64_t)dev.num_cus * (4 * c.wgs_per_cu - c.prefill_quarters));
  const int32_t p_half_items =
      small_prefill ? kFusedPrefillHalfItemsPerSlotSmall : kFusedPrefillHalfItemsPerSlotLarge;
  build_lists(pl->batch, dev, fused_p_slots, p_half_items, fused_d_waves, kFusedDecodeUnitsPerWave,
              t.prefill_kv_splits, t.decode_kv_splits, &pl->fused);
  // Sequential plan: each kernel has the whole GPU.
  pl->seq_is_fused = t.match_sequential == 1;
  if (!pl->seq_is_fused)
    build_lists(pl->batch, dev, slots, kSeqPrefillHalfItemsPerSlot, slots * kWavesPerWG, kSeqDecodeUnitsPerWave,
                t.prefill_kv_splits, t.decode_kv_splits, &pl->seq);
  const WorkLists& sq = pl->seq_is_fused ? pl->fused : pl->seq;
  pl->n_partials = std::max(pl->fused.n_partials, sq.n_partials);
  pl->trace_records = (t.flags & POD_FLAG_TRACE) ? pl->fused.n_p() + pl->fused.n_d() : 0;

  // workspace layout
  size_t off = 0;
  pl->off_counters = off;
  off = align_up(off + kCounterInts * sizeof(int32_t));
  auto place = [&](const WorkLists& w, DevLists& d) {
    d.p_items = off;
    off = align_up(off + w.p_items.size() * sizeof(int32_t));
    d.d_items = off;
    off = align_up(off + w.d_items.size() * sizeof(int32_t));
    d.m_tasks = off;
    off = align_up(off + w.m_tasks.size() * sizeof(int32_t));
  };
  place(pl->fused, pl->dl_fused);
  if (pl->seq_is_fused) pl->dl_seq = pl->dl_fused;
  else place(pl->seq, pl->dl_seq);
  pl->off_trace = off;
  off = align_up(off + (size_t)pl->trace_records * sizeof(pod_trace_record_t));
  pl->off_part_lse = off;
  off = align_up(off + (size_t)pl->n_partials * sizeof(float));
  pl->off_part_o = off;
  off = align_up(off + (size_t)pl->n_partials * kHeadDim * sizeof(uint16_t));
  pl->ws_bytes = off;
  return POD_OK;
}

pod_status_t query_device(pod_device_desc_t* dev, int* device) {
  hipError_t e = hipGetDevice(device);
  if (e != hipSuccess) return hip_err(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, *device);
  if (e != hipSuccess) return hip_err(e, "hipDeviceGetAttribute(CU count)");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, *device);
  if (e != hipSuccess) return hip_err(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_err(POD_ERR_UNSUPPORTED,
                   std::string("device is ") + prop.gcnArchName + ", library is built for gfx950");
  dev->num_cus = cus;
  dev->num_xcds = 8;   // MI355X: 8 accelerator dies, 32 CUs each
  return POD_OK;
}

template <class T>
pod_status_t upload(char* ws, size_t off, const std::vector<T>& v, hipStream_t s) {
  if (v.empty()) return POD_OK;
  hipError_t e = hipMemcpyAsync(ws + off, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice, s);
  return e == hipSuccess ? POD_OK : hip_err(e, "hipMemcpyAsync(work list)");
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pod_status_t check_tensors(const pod_attn_plan_s* pl, const pod_attn_tensors_t* t) {
  if (!pl) return set_err(POD_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!t) return set_err(POD_ERR_INVALID_ARGUMENT, "tensors is NULL");
  if (!pl->ws) return set_err(POD_ERR_INVALID_ARGUMENT, "plan has no workspace (host-only plan)");
  const bool has_p = !pl->batch.qo.empty(), has_d = !pl->batch.dkv.empty();
  auto need = [&](const void* p, const char* name) -> pod_status_t {
    if (!p) return set_err(POD_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
    if (!aligned16(p)) return set_err(POD_ERR_INVALID_ARGUMENT, std::string(name) + " is not 16-byte aligned");
    return POD_OK;
  };
  pod_status_t st;
  if (has_p || has_d) {
    if ((st = need(t->k, "k")) != POD_OK) return st;
    if ((st = need(t->v, "v")) != POD_OK) return st;
    if (pl->batch.params.kv_layout == POD_KV_PAGED) {
      if (!t->page_indptr || !t->page_indices)
        return set_err(POD_ERR_INVALID_ARGUMENT, "page_indptr/page_indices is NULL");
    } else if (!t->kv_indptr) {
      return set_err(POD_ERR_INVALID_ARGUMENT, "kv_indptr is NULL");
    }
  }
  if (has_p) {
    if ((st = need(t->q_prefill, "q_prefill")) != POD_OK) return st;
    if ((st = need(t->o_prefill, "o_prefill")) != POD_OK) return st;
  }
  if (has_d) {
    if ((st = need(t->q_decode, "q_decode")) != POD_OK) return st;
    if ((st = need(t->o_decode, "o_decode")) != POD_OK) return st;
  }
  return POD_OK;
}

int kv_mode_of(const pod_attn_plan_s* pl) {
  const auto& p = pl->batch.params;
  if (p.kv_layout != POD_KV_PAGED) return KV_CONTIG;
  return p.page_size >= 16 ? KV_PAGED_WIDE : KV_PAGED_NARROW;
}

// Counter blocks of a launch of `kind` on `stream`: alternate by launch
// parity, or the self-resetting block while the stream is being captured.
void pick_counters(pod_attn_plan_s* pl, int kind, hipStream_t stream, KernelArgs* a) {
  int32_t* base = (int32_t*)(pl->ws + pl->off_counters) + kind * kBlocksPerKind * kCtrBlockInts;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) cs = hipStreamCaptureStatusNone;
  if (cs != hipStreamCaptureStatusNone) {
    a->counters = base + 2 * kCtrBlockInts;
    a->counters_next = nullptr;
    a->self_reset = 1;
  } else {
    const int par = (int)(pl->launches[kind] & 1);
    a->counters = base + par * kCtrBlockInts;
    a->counters_next = base + (par ^ 1) * kCtrBlockInts;
    a->self_reset = 0;
  }
}

KernelArgs make_args(const pod_attn_plan_s* pl, const pod_attn_tensors_t* t, const WorkLists& w,
                     const DevLists& dl) {
  KernelArgs a;
  std::memset(&a, 0, sizeof(a));
  const auto& p = pl->batch.params;
  a.q_prefill = (const uint16_t*)t->q_prefill;
  a.q_decode = (const uint16_t*)t->q_decode;
  a.k = (const uint16_t*)t->k;
  a.v = (const uint16_t*)t->v;
  a.kv_indptr = t->kv_indptr;
  a.page_indptr = t->page_indptr;
  a.page_indices = t->page_indices;
  a.o_prefill = (uint16_t*)t->o_prefill;
  a.o_decode = (uint16_t*)t->o_decode;
  a.lse_prefill = t->lse_prefill;
  a.lse_decode = t->lse_decode;
  a.part_o = (uint16_t*)(pl->ws + pl->off_part_o);
  a.part_lse = (float*)(pl->ws + pl->off_part_lse);
  a.p_items = (const int32_t*)(pl->ws + dl.p_items);
  a.d_items = (const int32_t*)(pl->ws + dl.d_items);
  a.m_tasks = (const int32_t*)(pl->ws + dl.m_tasks);
  a.trace = nullptr;
  a.n_p = w.n_p();
  a.n_d = w.n_d();
  a.n_groups = w.n_groups();
  a.n_m = w.n_m();
  a.num_pools = (int32_t)w.pool_off.size() - 1;
  a.n_dq = std::min(kMaxDecodeQueues, 4 * a.num_pools);
  for (int i = 0; i <= a.num_pools && i <= kMaxPools; ++i) a.pool_off[i] = w.pool_off[i];
  a.hq = p.num_qo_heads;
  a.hkv = p.num_kv_heads;
  a.group = p.num_qo_heads / p.num_kv_heads;
  a.p_heads = prefill_heads(a.group);
  int sh = 0;
  if (p.kv_layout == POD_KV_PAGED)
    while ((1 << sh) < p.page_size) ++sh;
  a.page_shift = sh;
  a.causal = p.causal;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  a.wgs_per_cu = pl->choice.wgs_per_cu;
  a.prefill_quarters = pl->choice.prefill_quarters;
  a.sched_mode = pl->choice.sched_mode;
  return a;
}

}  // namespace

extern "C" {

const char* pod_attn_last_error(void) { return g_err.c_str(); }

pod_status_t pod_attn_plan_host(const pod_attn_params_t* params, int32_t num_prefill,
                                const int32_t* prefill_qo_len, const int32_t* prefill_kv_len,
                                int32_t num_decode, const int32_t* decode_kv_len,
                                const pod_attn_tuning_t* tuning, const pod_device_desc_t* device,
                                pod_attn_plan_t* out_plan) {
  if (!out_plan) return set_err(POD_ERR_INVALID_ARGUMENT, "out_plan is NULL");
  *out_plan = nullptr;
  if (!device) return set_err(POD_ERR_INVALID_ARGUMENT, "device is NULL");
  pod_attn_plan_s* pl = new (std::nothrow) pod_attn_plan_s();
  if (!pl) return set_err(POD_ERR_INTERNAL, "out of host memory");
  pod_status_t st;
  try {
    st = build_plan(params, num_prefill, prefill_qo_len, prefill_kv_len, num_decode,
                    decode_kv_len, tuning, *device, pl);
  } catch (const std::exception& ex) {
    st = set_err(POD_ERR_INTERNAL, ex.what());
  }
  if (st != POD_OK) {
    delete pl;
    return st;
  }
  *out_plan = pl;
  return POD_OK;
}

pod_status_t pod_attn_plan(const pod_attn_params_t* params, int32_t num_prefill,
                           const int32_t* prefill_qo_len, const int32_t* prefill_kv_len,
                           int32_t num_decode, const int32_t* decode_kv_len,
                           const pod_attn_tuning_t* tuning, void* workspace,
                           size_t workspace_bytes, size_t* workspace_needed, hipStream_t stream,
                           pod_attn_plan_t* out_plan) {
  if (out_plan) *out_plan = nullptr;
  if (!workspace_needed && !workspace)
    return set_err(POD_ERR_INVALID_ARGUMENT, "workspace and workspace_needed are both NULL");
  pod_device_desc_t dev;
  int device = -1;
  pod_status_t st = query_device(&dev, &device);
  if (st != POD_OK) return st;
  pod_attn_plan_s* pl = new (std::nothrow) pod_attn_plan_s();
  if (!pl) return set_err(POD_ERR_INTERNAL, "out of host memory");
  try {
    st = build_plan(params, num_prefill, prefill_qo_len, prefill_kv_len, num_decode,
                    decode_kv_len, tuning, dev, pl);
  } catch (const std::exception& ex) {
    st = set_err(POD_ERR_INTERNAL, ex.what());
  }
  if (st != POD_OK) {
    delete pl;
    return st;
  }
  if (workspace_needed) *workspace_needed = pl->ws_bytes;
  if (!workspace) {
    delete pl;
    return POD_OK;
  }
  if (!out_plan) {
    delete pl;
    return set_err(POD_ERR_INVALID_ARGUMENT, "out_plan is NULL");
  }
  if (workspace_bytes < pl->ws_bytes) {
    char buf[128];
    std::snprintf(buf, sizeof(buf), "workspace has %zu bytes, plan needs %zu", workspace_bytes,
                  pl->ws_bytes);
    delete pl;
    return set_err(POD_ERR_WORKSPACE_TOO_SMALL, buf);
  }
  if (!aligned16(workspace)) {
    delete pl;
    return set_err(POD_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
  }
  pl->ws = (char*)workspace;
  pl->device = device;
  hipError_t e = hipMemsetAsync(pl->ws + pl->off_counters, 0, kCounterInts * sizeof(int32_t), stream);
  if (e != hipSuccess) {
    delete pl;
    return hip_err(e, "hipMemsetAsync(counters)");
  }
  auto up = [&](const WorkLists& w, const DevLists& d) -> pod_status_t {
    pod_status_t s2;
    if ((s2 = upload(pl->ws, d.p_items, w.p_items, stream)) != POD_OK) return s2;
    if ((s2 = upload(pl->ws, d.d_items, w.d_items, stream)) != POD_OK) return s2;
    return upload(pl->ws, d.m_tasks, w.m_tasks, stream);
  };
  if ((st = up(pl->fused, pl->dl_fused)) != POD_OK || (!pl->seq_is_fused && (st = up(pl->seq, pl->dl_seq)) != POD_OK)) {
    delete pl;
    return st;
  }
  *out_plan = pl;
  return POD_OK;
}

pod_status_t pod_attn_run_events(pod_attn_plan_t pl, const pod_attn_tensors_t* t,
                                 hipStream_t stream, hipEvent_t before_fused,
                                 hipEvent_t after_fused) {
  pod_status_t st = check_tensors(pl, t);
  if (st != POD_OK) return st;
  const WorkLists& w = pl->fused;
  KernelArgs a = make_args(pl, t, w, pl->dl_fused);
  pick_counters(pl, kKindFused, stream, &a);
  if (pl->trace_records) a.trace = (pod_trace_record_t*)(pl->ws + pl->off_trace);
  // persistent: wgs_per_cu workgroups per CU, fewer when there are fewer units
  const int64_t slots = (int64_t)pl->dev.num_cus * pl->choice.wgs_per_cu;
  const int grid = (int)std::min<int64_t>(slots, (int64_t)w.n_p() + w.n_groups());
  hipError_t e;
  if (before_fused && (e = hipEventRecord(before_fused, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(before_fused)");
  if (grid > 0) {
    e = launch_fused(a, kv_mode_of(pl), grid, stream);
    if (e != hipSuccess) return hip_err(e, "fused kernel launch");
    if (!a.self_reset) ++pl->launches[kKindFused];
  }
  if (after_fused && (e = hipEventRecord(after_fused, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(after_fused)");
  if (w.n_m() > 0) {
    e = launch_merge(a, (w.n_m() + kMergeTasksPerWG - 1) / kMergeTasksPerWG, stream);
    if (e != hipSuccess) return hip_err(e, "merge kernel launch");
  }
  return POD_OK;
}

pod_status_t pod_attn_run(pod_attn_plan_t pl, const pod_attn_tensors_t* t, hipStream_t stream) {
  return pod_attn_run_events(pl, t, stream, nullptr, nullptr);
}

pod_status_t pod_attn_sequential_run(pod_attn_plan_t pl, const pod_attn_tensors_t* t,
                                     hipStream_t stream) {
  pod_status_t st = check_tensors(pl, t);
  if (st != POD_OK) return st;
  const WorkLists& w = pl->seq_is_fused ? pl->fused : pl->seq;
  KernelArgs a = make_args(pl, t, w, pl->dl_seq);
  pick_counters(pl, kKindSeq, stream, &a);
  // the trace is indexed by the fused lists' units, so only a plan-matched
  // sequential run records it
  if (pl->trace_records && pl->seq_is_fused)
    a.trace = (pod_trace_record_t*)(pl->ws + pl->off_trace);
  const int kvm = kv_mode_of(pl);
  if (w.n_p() > 0) {
    hipError_t e = launch_prefill(a, kvm, w.n_p(), stream);
    if (e != hipSuccess) return hip_err(e, "prefill kernel launch");
    if (!a.self_reset) ++pl->launches[kKindSeq];
  }
  if (w.n_groups() > 0) {
    hipError_t e = launch_decode(a, kvm, w.n_groups(), stream);
    if (e != hipSuccess) return hip_err(e, "decode kernel launch");
  }
  if (w.n_m() > 0) {
    hipError_t e = launch_merge(a, (w.n_m() + kMergeTasksPerWG - 1) / kMergeTasksPerWG, stream);
    if (e != hipSuccess) return hip_err(e, "merge kernel launch");
  }
  return POD_OK;
}

pod_status_t pod_attn_plan_info(pod_attn_plan_t pl, pod_attn_plan_info_t* out) {
  if (!pl || !out) return set_err(POD_ERR_INVALID_ARGUMENT, "NULL argument");
  const WorkLists& sq = pl->seq_is_fused ? pl->fused : pl->seq;
  out->prefill_items = pl->fused.n_p();
  out->decode_items = pl->fused.n_d();
  out->decode_groups = pl->fused.n_groups();
  out->merge_tasks = pl->fused.n_m();
  out->seq_prefill_items = sq.n_p();
  out->seq_decode_items = sq.n_d();
  out->seq_merge_tasks = sq.n_m();
  out->prefill_splits_max = pl->fused.p_splits_max;
  out->decode_splits_max = pl->fused.d_splits_max;
  out->wgs_per_cu = pl->choice.wgs_per_cu;
  out->prefill_quarters_per_cu = pl->choice.prefill_quarters;
  out->sched_mode = pl->choice.sched_mode;
  out->num_partials = pl->n_partials;
  out->trace_records = pl->trace_records;
  out->workspace_bytes = pl->ws_bytes;
  return POD_OK;
}

pod_status_t pod_attn_plan_export(pod_attn_plan_t pl, int32_t which, int32_t* dst, size_t n,
                                  size_t* count) {
  if (!pl || !count) return set_err(POD_ERR_INVALID_ARGUMENT, "NULL argument");
  const WorkLists& sq = pl->seq_is_fused ? pl->fused : pl->seq;
  const std::vector<int32_t>* v = nullptr;
  switch (which) {
    case 0: v = &pl->fused.p_items; break;
    case 1: v = &pl->fused.d_items; break;
    case 2: v = &pl->fused.m_tasks; break;
    case 3: v = &sq.p_items; break;
    case 4: v = &sq.d_items; break;
    case 5: v = &sq.m_tasks; break;
    case 6: v = &pl->fused.pool_off; break;
    case 7: v = &sq.pool_off; break;
    default: return set_err(POD_ERR_INVALID_ARGUMENT, "unknown list id");
  }
  *count = v->size();
  if (dst) std::memcpy(dst, v->data(), std::min(n, v->size()) * sizeof(int32_t));
  return POD_OK;
}

pod_status_t pod_attn_read_trace(pod_attn_plan_t pl, pod_trace_record_t* dst, size_t n,
                                 size_t* count, hipStream_t stream) {
  if (!pl || !count) return set_err(POD_ERR_INVALID_ARGUMENT, "NULL argument");
  if (!pl->ws) return set_err(POD_ERR_INVALID_ARGUMENT, "plan has no workspace");
  *count = (size_t)pl->trace_records;
  if (!dst || pl->trace_records == 0) return POD_OK;
  const size_t m = std::min(n, (size_t)pl->trace_records);
  hipError_t e = hipMemcpyAsync(dst, pl->ws + pl->off_trace, m * sizeof(pod_trace_record_t),
                                hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync(trace)");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_err(e, "hipStreamSynchronize");
  return POD_OK;
}

void pod_attn_plan_destroy(pod_attn_plan_t pl) { delete pl; }

pod_status_t pod_attn_probe_hwid(int32_t num_blocks, int32_t* out, hipStream_t stream) {
  if (num_blocks < 1 || !out) return set_err(POD_ERR_INVALID_ARGUMENT, "bad probe arguments");
  hipError_t e = launch_probe(out, num_blocks, stream);
  return e == hipSuccess ? POD_OK : hip_err(e, "probe kernel launch");
}

}  // extern "C"
