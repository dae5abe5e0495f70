// C ABI of libpod_attn.so (declared in include/pod_attn.h).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
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
  WorkLists bp;                // batched-prefill comparator (POD_FLAG_BATCHED_PREFILL)
  bool seq_is_fused = false;
  bool has_bp = false;
  bool has_prefix = false;     // shared-prefix plan: `fused` holds the packed lists
  std::vector<int32_t> members;   // shared-prefix plan: decode index of each group member
  size_t off_members = 0;
  int32_t n_partials = 0;
  int32_t trace_records = 0;
  // workspace layout (bytes)
  size_t off_counters = 0, off_trace = 0, off_part_lse = 0, off_part_o = 0;
  DevLists dl_fused, dl_seq, dl_bp;
  // two-stream comparator: fork / join events (created on first use)
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipStream_t aux = nullptr;   // two-stream plans: the device's second stream (not owned)
  uint64_t launches[2] = {0, 0};   // successful launches per kind (counter parity)
  size_t ws_bytes = 0;
  char* ws = nullptr;          // caller-owned device buffer (NULL: host-only plan)
  int device = -1;
  ~pod_attn_plan_s() {
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
  }
};

namespace {

pod_status_t layout_workspace(pod_attn_plan_s* pl);

// The second stream pod_attn_run uses for plans that run the prefill and
// decode kernels at once: one per device, created (default priority,
// non-blocking) by the first such plan on that device, with the device
// current, and kept until the process ends.  Plans share it: their decode
// kernels queue on it in the order their runs enqueue them.
hipError_t aux_stream(int device, hipStream_t* out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static hipStream_t streams[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[device]) {
    hipStream_t s = nullptr;
    const hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    streams[device] = s;
  }
  *out = streams[device];
  return hipSuccess;
}

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
  c.one_unit = (t.flags & POD_FLAG_ONE_UNIT_PER_WG) != 0;
  if (c.sched_mode == POD_SCHED_ORDERED) {
    // one queue, prefill units first: each part has the whole GPU in turn,
    // so the lists are sized as the sequential kernels' are
    build_lists(pl->batch, dev, slots, kSeqPrefillHalfItemsPerSlot, slots * kWavesPerWG,
                kSeqDecodeUnitsPerWave, t.prefill_kv_splits, t.decode_kv_splits, &pl->fused);
  } else {
    const int64_t fused_p_slots = small_prefill ? p_slots_coloc : slots;
    const int64_t fused_d_waves = std::max<int64_t>(
        kWavesPerWG, (int64_t)dev.num_cus * (4 * c.wgs_per_cu - c.prefill_quarters));
    const int32_t p_half_items =
        small_prefill ? kFusedPrefillHalfItemsPerSlotSmall : kFusedPrefillHalfItemsPerSlotLarge;
    build_lists(pl->batch, dev, fused_p_slots, p_half_items, fused_d_waves,
                kFusedDecodeUnitsPerWave, t.prefill_kv_splits, t.decode_kv_splits, &pl->fused);
  }
  // automatic launch shape (kOneUnitSlotsFactor): a small batch runs one
  // workgroup per unit.  With several prefill requests each workgroup takes
  // its role from its CU index, as the persistent CU partition does, over
  // the same lists; with one, from its CU's ticket, over lists rebuilt for
  // the co-location share (measurements at kOneUnitSlotsFactor)
  if (t.sched_mode == POD_SCHED_AUTO && !c.one_unit && np > 1 &&
      (int64_t)pl->fused.n_p() + pl->fused.n_groups() <= kOneUnitSlotsFactor * slots) {
    c.one_unit = true;
  } else if (t.sched_mode == POD_SCHED_AUTO && !c.one_unit &&
             (int64_t)pl->fused.n_p() + pl->fused.n_groups() <= kOneUnitSlotsFactor * slots) {
    c.sched_mode = POD_SCHED_COLOCATE;
    c.one_unit = true;
    if (t.prefill_quarters_per_cu < 0)
      c.prefill_quarters = auto_prefill_quarters(pl->batch, c.wgs_per_cu, c.sched_mode);
    const int64_t p_slots = std::max<int64_t>(1, (int64_t)dev.num_cus * c.prefill_quarters / 4);
    const int64_t d_waves = std::max<int64_t>(
        kWavesPerWG, (int64_t)dev.num_cus * (4 * c.wgs_per_cu - c.prefill_quarters));
    build_lists(pl->batch, dev, small_prefill ? p_slots : slots,
                small_prefill ? kFusedPrefillHalfItemsPerSlotSmall
                              : kFusedPrefillHalfItemsPerSlotLarge,
                d_waves, kFusedDecodeUnitsPerWave, t.prefill_kv_splits, t.decode_kv_splits,
                &pl->fused);
  }
  // Sequential plan: each kernel has the whole GPU.
  pl->seq_is_fused = t.match_sequential == 1;
  if (!pl->seq_is_fused)
    build_lists(pl->batch, dev, slots, kSeqPrefillHalfItemsPerSlot, slots * kWavesPerWG, kSeqDecodeUnitsPerWave,
                t.prefill_kv_splits, t.decode_kv_splits, &pl->seq);
  // Batched-prefill comparator: every request through the prefill kernel,
  // split like the sequential plan's prefill.
  pl->has_bp = (t.flags & POD_FLAG_BATCHED_PREFILL) != 0;
  if (pl->has_bp)
    build_lists(pl->batch, dev, slots, kSeqPrefillHalfItemsPerSlot, 0, 1, t.prefill_kv_splits, 0,
                &pl->bp, /*decodes_as_prefill=*/true);
  pl->trace_records = (t.flags & POD_FLAG_TRACE) ? pl->fused.n_p() + pl->fused.n_d() : 0;
  // MHA with a small prefill share: the two kernels back to back
  // (kMhaSequentialShare); only when the caller left the mode to the planner,
  // and not for the small batches that run one workgroup per unit (launch
  // bound: the tiny batch measured 0.99-1.04x fused against sequential)
  // GQA with several prefill requests and a small prefill share: the two
  // kernels at once on two streams (kGqaStreamsShare)
  if (t.sched_mode == POD_SCHED_AUTO && !c.one_unit && np > 0 && nd > 0) {
    const double share = prefill_share_estimate(pl->batch);
    if (params->num_qo_heads == params->num_kv_heads && share < kMhaSequentialShare)
      c.runs_sequential = 1;
    else if (params->num_qo_heads > params->num_kv_heads && np > 1 && share < kGqaStreamsShare)
      c.runs_sequential = 2;
  }
  return layout_workspace(pl);
}

// Workspace layout of a plan: counters, the work lists, trace, partials.
// Refuses lists whose split partials outgrow their int32 indices.
pod_status_t layout_workspace(pod_attn_plan_s* pl) {
  const WorkLists& sq = pl->seq_is_fused ? pl->fused : pl->seq;
  if (pl->fused.n_partials < 0 || sq.n_partials < 0 || pl->bp.n_partials < 0)
    return set_err(POD_ERR_UNSUPPORTED,
                   "the plan needs more than 2^31 - 1 split partials (force fewer KV splits or "
                   "plan a smaller batch)");
  pl->n_partials = std::max(std::max(pl->fused.n_partials, sq.n_partials), pl->bp.n_partials);
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
  if (pl->has_bp) place(pl->bp, pl->dl_bp);
  pl->off_members = off;
  off = align_up(off + pl->members.size() * sizeof(int32_t));
  pl->off_trace = off;
  off = align_up(off + (size_t)pl->trace_records * sizeof(pod_trace_record_t));
  pl->off_part_lse = off;
  off = align_up(off + (size_t)pl->n_partials * sizeof(float));
  pl->off_part_o = off;
  off = align_up(off + (size_t)pl->n_partials * kHeadDim * sizeof(float));
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
  if (pl->batch.params.kv_dtype == POD_KV_FP8_E4M3 && (has_p || has_d) &&
      (!t->k_scale || !t->v_scale))
    return set_err(POD_ERR_INVALID_ARGUMENT, "k_scale/v_scale is NULL (FP8 KV cache)");
  return POD_OK;
}

bool is_fp8(const pod_attn_plan_s* pl) { return pl->batch.params.kv_dtype == POD_KV_FP8_E4M3; }

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
  a.k_scale = t->k_scale;
  a.v_scale = t->v_scale;
  a.kv_fp8 = p.kv_dtype == POD_KV_FP8_E4M3;
  a.d_members = (const int32_t*)(pl->ws + pl->off_members);
  a.pack_rpr = std::min(p.num_qo_heads / p.num_kv_heads, kDecodeRows);
  a.part_o = (float*)(pl->ws + pl->off_part_o);
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
  a.one_unit = pl->choice.one_unit ? 1 : 0;
  a.n_preq = (int32_t)pl->batch.qo.size();
  a.merge_splits = 0;
  a.merge_lse_scale = 1.0f;
  return a;
}

pod_status_t launch_merge_of(const KernelArgs& a, const WorkLists& w, hipStream_t stream) {
  if (w.n_m() == 0) return POD_OK;
  hipError_t e = launch_merge(a, (w.n_m() + kMergeTasksPerWG - 1) / kMergeTasksPerWG, stream);
  return e == hipSuccess ? POD_OK : hip_err(e, "merge kernel launch");
}

// The device half of a plan call: reports the workspace size, or takes the
// caller's workspace, zeroes the counters and uploads the work lists on
// `stream`.  Consumes `pl` (deleted unless it becomes *out_plan).
// A decode-only plan for queries packed by shared prefix ([PAT] abstract):
// the ordinary decode lists (the unshared baseline) for the sequential and
// streams paths, the packed lists in place of the fused ones.
pod_status_t build_prefix_plan(const pod_attn_params_t* params, int32_t nd, const int32_t* dkv,
                               const int32_t* prefix_group, int32_t num_groups,
                               const int32_t* prefix_len, const pod_attn_tuning_t* tuning,
                               const pod_device_desc_t& dev, pod_attn_plan_s* pl) {
  if (!params) return set_err(POD_ERR_INVALID_ARGUMENT, "params is NULL");
  if (params->kv_layout != POD_KV_PAGED || params->kv_dtype != POD_KV_BF16)
    return set_err(POD_ERR_UNSUPPORTED, "shared-prefix plans need a paged bf16 cache");
  if (tuning && (tuning->flags & POD_FLAG_BATCHED_PREFILL))
    return set_err(POD_ERR_UNSUPPORTED, "no batched-prefill comparator for shared-prefix plans");
  if (num_groups < 0 || (num_groups > 0 && !prefix_len) || (nd > 0 && (!prefix_group || !dkv)))
    return set_err(POD_ERR_INVALID_ARGUMENT, "prefix group arrays are NULL or num_groups < 0");
  std::vector<int32_t> group_of(prefix_group, prefix_group + std::max(0, nd));
  std::vector<int32_t> plen(prefix_len, prefix_len + num_groups);
  for (int32_t i = 0; i < nd; ++i) {
    const int32_t gi = group_of[i];
    if (gi < -1 || gi >= num_groups)
      return set_err(POD_ERR_INVALID_ARGUMENT, "prefix_group entry out of range");
    if (gi >= 0 && (plen[gi] < 1 || params->page_size < 1 || plen[gi] % params->page_size != 0 ||
                    plen[gi] > dkv[i]))
      return set_err(POD_ERR_INVALID_ARGUMENT,
                     "a shared prefix must be whole pages, >= 1 token and no longer than any "
                     "member's kv_len");
  }
  pod_attn_tuning_t t{};
  t.prefill_quarters_per_cu = -1;
  if (tuning) t = *tuning;
  t.match_sequential = 0;
  t.flags &= ~(POD_FLAG_TRACE | POD_FLAG_ONE_UNIT_PER_WG);
  try {
    pod_status_t st = build_plan(params, 0, nullptr, nullptr, nd, dkv, &t, dev, pl);
    if (st != POD_OK) return st;
    const int64_t waves = (int64_t)dev.num_cus * pl->choice.wgs_per_cu * kWavesPerWG;
    build_prefix_lists(pl->batch, group_of, plen, waves, t.decode_kv_splits, &pl->fused,
                       &pl->members);
    pl->has_prefix = true;
    pl->trace_records = 0;
    if ((st = layout_workspace(pl)) != POD_OK) return st;
  } catch (const std::exception& ex) {
    return set_err(POD_ERR_INTERNAL, ex.what());
  }
  return POD_OK;
}

pod_status_t finish_device_plan(pod_attn_plan_s* pl, int device, void* workspace,
                                size_t workspace_bytes, size_t* workspace_needed,
                                hipStream_t stream, pod_attn_plan_t* out_plan) {
  pod_status_t st;
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
  if (pl->choice.runs_sequential == 2) {
    const hipError_t es = aux_stream(device, &pl->aux);
    if (es != hipSuccess) {
      delete pl;
      return hip_err(es, "hipStreamCreateWithFlags (second stream)");
    }
  }
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
  if ((st = up(pl->fused, pl->dl_fused)) != POD_OK ||
      (!pl->seq_is_fused && (st = up(pl->seq, pl->dl_seq)) != POD_OK) ||
      (pl->has_bp && (st = up(pl->bp, pl->dl_bp)) != POD_OK) ||
      (st = upload(pl->ws, pl->off_members, pl->members, stream)) != POD_OK) {
    delete pl;
    return st;
  }
  *out_plan = pl;
  return POD_OK;
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

namespace {

// pod_attn_plan; with `no_streams` a batch the planner would run on two
// streams runs the fused launch instead (no stream is created).
pod_status_t plan_on_device(const pod_attn_params_t* params, int32_t num_prefill,
                            const int32_t* prefill_qo_len, const int32_t* prefill_kv_len,
                            int32_t num_decode, const int32_t* decode_kv_len,
                            const pod_attn_tuning_t* tuning, void* workspace,
                            size_t workspace_bytes, size_t* workspace_needed, hipStream_t stream,
                            pod_attn_plan_t* out_plan, bool no_streams) {
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
  if (no_streams && pl->choice.runs_sequential == 2) pl->choice.runs_sequential = 0;
  return finish_device_plan(pl, device, workspace, workspace_bytes, workspace_needed, stream,
                            out_plan);
}

}  // namespace

pod_status_t pod_attn_plan(const pod_attn_params_t* params, int32_t num_prefill,
                           const int32_t* prefill_qo_len, const int32_t* prefill_kv_len,
                           int32_t num_decode, const int32_t* decode_kv_len,
                           const pod_attn_tuning_t* tuning, void* workspace,
                           size_t workspace_bytes, size_t* workspace_needed, hipStream_t stream,
                           pod_attn_plan_t* out_plan) {
  return plan_on_device(params, num_prefill, prefill_qo_len, prefill_kv_len, num_decode,
                        decode_kv_len, tuning, workspace, workspace_bytes, workspace_needed,
                        stream, out_plan, false);
}

pod_status_t pod_attn_plan_shared_prefix(const pod_attn_params_t* params, int32_t num_decode,
                                         const int32_t* decode_kv_len,
                                         const int32_t* prefix_group, int32_t num_groups,
                                         const int32_t* prefix_len,
                                         const pod_attn_tuning_t* tuning, void* workspace,
                                         size_t workspace_bytes, size_t* workspace_needed,
                                         hipStream_t stream, pod_attn_plan_t* out_plan) {
  if (out_plan) *out_plan = nullptr;
  if (!workspace_needed && !workspace)
    return set_err(POD_ERR_INVALID_ARGUMENT, "workspace and workspace_needed are both NULL");
  pod_device_desc_t dev;
  int device = -1;
  pod_status_t st = query_device(&dev, &device);
  if (st != POD_OK) return st;
  pod_attn_plan_s* pl = new (std::nothrow) pod_attn_plan_s();
  if (!pl) return set_err(POD_ERR_INTERNAL, "out of host memory");
  st = build_prefix_plan(params, num_decode, decode_kv_len, prefix_group, num_groups, prefix_len,
                         tuning, dev, pl);
  if (st != POD_OK) {
    delete pl;
    return st;
  }
  return finish_device_plan(pl, device, workspace, workspace_bytes, workspace_needed, stream,
                            out_plan);
}

pod_status_t pod_attn_plan_shared_prefix_host(const pod_attn_params_t* params,
                                              int32_t num_decode, const int32_t* decode_kv_len,
                                              const int32_t* prefix_group, int32_t num_groups,
                                              const int32_t* prefix_len,
                                              const pod_attn_tuning_t* tuning,
                                              const pod_device_desc_t* device,
                                              pod_attn_plan_t* out_plan) {
  if (!out_plan) return set_err(POD_ERR_INVALID_ARGUMENT, "out_plan is NULL");
  *out_plan = nullptr;
  if (!device) return set_err(POD_ERR_INVALID_ARGUMENT, "device is NULL");
  pod_attn_plan_s* pl = new (std::nothrow) pod_attn_plan_s();
  if (!pl) return set_err(POD_ERR_INTERNAL, "out of host memory");
  const pod_status_t st = build_prefix_plan(params, num_decode, decode_kv_len, prefix_group,
                                            num_groups, prefix_len, tuning, *device, pl);
  if (st != POD_OK) {
    delete pl;
    return st;
  }
  *out_plan = pl;
  return POD_OK;
}

pod_status_t pod_attn_plan_scratch(const pod_attn_params_t* params, int32_t num_prefill,
                                   const int32_t* prefill_qo_len, const int32_t* prefill_kv_len,
                                   int32_t num_decode, const int32_t* decode_kv_len,
                                   const pod_attn_tuning_t* tuning, hipStream_t stream,
                                   pod_attn_plan_t* out_plan) {
  if (!out_plan) return set_err(POD_ERR_INVALID_ARGUMENT, "out_plan is NULL");
  *out_plan = nullptr;
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_err(e, "hipGetDevice");
  void* ws = nullptr;
  if ((e = scratch_address(device, &ws)) != hipSuccess)
    return hip_err(e, "hipGetSymbolAddress(scratch)");
  size_t need = 0;
  // the two-stream route creates a stream: plans made here run those
  // batches as one fused launch instead
  pod_status_t st = plan_on_device(params, num_prefill, prefill_qo_len, prefill_kv_len,
                                   num_decode, decode_kv_len, tuning, nullptr, 0, &need, stream,
                                   nullptr, true);
  if (st != POD_OK) return st;
  if (need > kScratchBytes) {
    char buf[200];
    std::snprintf(buf, sizeof(buf),
                  "plan needs %zu bytes of workspace; the static scratch holds %zu (use "
                  "pod_attn_plan with a caller workspace)", need, kScratchBytes);
    return set_err(POD_ERR_WORKSPACE_TOO_SMALL, buf);
  }
  return plan_on_device(params, num_prefill, prefill_qo_len, prefill_kv_len, num_decode,
                        decode_kv_len, tuning, ws, kScratchBytes, &need, stream, out_plan, true);
}

namespace {

// Prefill kernel, decode kernel, merge on one stream with the sequential
// plan's lists; `before` / `after` (may be NULL) are recorded around the
// kernels that precede the merge.
pod_status_t run_sequential(pod_attn_plan_t pl, const pod_attn_tensors_t* t, hipStream_t stream,
                            hipEvent_t before, hipEvent_t after) {
  const WorkLists& w = pl->seq_is_fused ? pl->fused : pl->seq;
  KernelArgs a = make_args(pl, t, w, pl->dl_seq);
  pick_counters(pl, kKindSeq, stream, &a);
  // the trace is indexed by the fused lists' units, so only a plan-matched
  // sequential run records it
  if (pl->trace_records && pl->seq_is_fused)
    a.trace = (pod_trace_record_t*)(pl->ws + pl->off_trace);
  const int kvm = kv_mode_of(pl);
  hipError_t e;
  if (before && (e = hipEventRecord(before, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(before)");
  if (w.n_p() > 0) {
    e = launch_prefill(a, kvm, w.n_p(), stream);
    if (e != hipSuccess) return hip_err(e, "prefill kernel launch");
    if (!a.self_reset) ++pl->launches[kKindSeq];
  }
  if (w.n_groups() > 0) {
    e = is_fp8(pl) ? launch_decode_fp8(a, kvm, w.n_groups(), stream)
                   : launch_decode(a, kvm, w.n_groups(), stream);
    if (e != hipSuccess) return hip_err(e, "decode kernel launch");
  }
  if (after && (e = hipEventRecord(after, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(after)");
  return launch_merge_of(a, w, stream);
}

}  // namespace

namespace {

// Prefill kernel on `stream`, decode kernel on `decode_stream` (forked from
// and joined back to `stream` by events), then the merge on `stream`;
// `before` / `after` (may be NULL) are recorded on `stream` around the two
// kernels.  Only the prefill kernel claims work through the counters (the
// decode kernel runs one group per workgroup of its grid), so the two
// kernels running at once share the sequential kind's counter block safely,
// captured (self-resetting) or not.
pod_status_t run_streams(pod_attn_plan_t pl, const pod_attn_tensors_t* t, hipStream_t stream,
                         hipStream_t decode_stream, hipEvent_t before, hipEvent_t after) {
  const WorkLists& w = pl->seq_is_fused ? pl->fused : pl->seq;
  KernelArgs a = make_args(pl, t, w, pl->dl_seq);
  pick_counters(pl, kKindSeq, stream, &a);
  hipError_t e;
  for (hipEvent_t* ev : {&pl->ev_fork, &pl->ev_join})
    if (!*ev && (e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess)
      return hip_err(e, "hipEventCreateWithFlags");
  if (before && (e = hipEventRecord(before, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(before)");
  // the decode stream starts after the work already enqueued on `stream`
  if ((e = hipEventRecord(pl->ev_fork, stream)) != hipSuccess) return hip_err(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(decode_stream, pl->ev_fork, 0)) != hipSuccess)
    return hip_err(e, "hipStreamWaitEvent");
  const int kvm = kv_mode_of(pl);
  if (w.n_p() > 0) {
    if ((e = launch_prefill(a, kvm, w.n_p(), stream)) != hipSuccess)
      return hip_err(e, "prefill kernel launch");
    if (!a.self_reset) ++pl->launches[kKindSeq];
  }
  if (w.n_groups() > 0 &&
      (e = is_fp8(pl) ? launch_decode_fp8(a, kvm, w.n_groups(), decode_stream)
                      : launch_decode(a, kvm, w.n_groups(), decode_stream)) != hipSuccess)
    return hip_err(e, "decode kernel launch");
  // join: the merge (and whatever the caller enqueues next) waits for both
  if ((e = hipEventRecord(pl->ev_join, decode_stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(stream, pl->ev_join, 0)) != hipSuccess)
    return hip_err(e, "hipStreamWaitEvent");
  if (after && (e = hipEventRecord(after, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(after)");
  return launch_merge_of(a, w, stream);
}

}  // namespace

pod_status_t pod_attn_run_events(pod_attn_plan_t pl, const pod_attn_tensors_t* t,
                                 hipStream_t stream, hipEvent_t before_fused,
                                 hipEvent_t after_fused) {
  pod_status_t st = check_tensors(pl, t);
  if (st != POD_OK) return st;
  // A batch of one kind (no decodes, or no prefill) has nothing to overlap:
  // it runs the one kernel it needs with the sequential plan's lists, as the
  // fused launch would only hold units of that kind.  (Traced plans keep the
  // fused launch: the trace is indexed by its units.)
  if (!pl->has_prefix && !pl->trace_records && pl->choice.runs_sequential == 2 && pl->aux &&
      pl->fused.n_p() > 0 && pl->fused.n_d() > 0 && stream != pl->aux)
    return run_streams(pl, t, stream, pl->aux, before_fused, after_fused);
  if (!pl->has_prefix && !pl->trace_records &&
      (pl->fused.n_p() == 0 || pl->fused.n_d() == 0 || pl->choice.runs_sequential))
    return run_sequential(pl, t, stream, before_fused, after_fused);
  const WorkLists& w = pl->fused;
  KernelArgs a = make_args(pl, t, w, pl->dl_fused);
  pick_counters(pl, kKindFused, stream, &a);
  if (pl->trace_records) a.trace = (pod_trace_record_t*)(pl->ws + pl->off_trace);
  // persistent: wgs_per_cu workgroups per CU, fewer when there are fewer
  // units; or one workgroup per unit
  const int64_t slots = (int64_t)pl->dev.num_cus * pl->choice.wgs_per_cu;
  const int64_t units = (int64_t)w.n_p() + w.n_groups();
  const int grid = (int)(a.one_unit ? units : std::min<int64_t>(slots, units));
  hipError_t e;
  if (before_fused && (e = hipEventRecord(before_fused, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(before_fused)");
  if (pl->has_prefix) {
    // shared-prefix plan: packed prefix units and suffix units, then the merge
    const int pgrid = w.n_p() + w.n_groups();
    if (pgrid > 0 && (e = launch_decode_pack(a, kv_mode_of(pl), pgrid, stream)) != hipSuccess)
      return hip_err(e, "packed decode kernel launch");
  } else if (grid > 0) {
    e = launch_fused(a, kv_mode_of(pl), grid, stream);
    if (e != hipSuccess) return hip_err(e, "fused kernel launch");
    if (!a.self_reset) ++pl->launches[kKindFused];
  }
  if (after_fused && (e = hipEventRecord(after_fused, stream)) != hipSuccess)
    return hip_err(e, "hipEventRecord(after_fused)");
  return launch_merge_of(a, w, stream);
}

pod_status_t pod_attn_run(pod_attn_plan_t pl, const pod_attn_tensors_t* t, hipStream_t stream) {
  return pod_attn_run_events(pl, t, stream, nullptr, nullptr);
}

pod_status_t pod_attn_sequential_run(pod_attn_plan_t pl, const pod_attn_tensors_t* t,
                                     hipStream_t stream) {
  pod_status_t st = check_tensors(pl, t);
  if (st != POD_OK) return st;
  return run_sequential(pl, t, stream, nullptr, nullptr);
}

pod_status_t pod_attn_streams_run(pod_attn_plan_t pl, const pod_attn_tensors_t* t,
                                  hipStream_t stream, hipStream_t decode_stream) {
  pod_status_t st = check_tensors(pl, t);
  if (st != POD_OK) return st;
  if (decode_stream == stream)
    return set_err(POD_ERR_INVALID_ARGUMENT, "decode_stream must differ from stream");
  return run_streams(pl, t, stream, decode_stream, nullptr, nullptr);
}

pod_status_t pod_attn_batched_prefill_run(pod_attn_plan_t pl, const pod_attn_tensors_t* t,
                                          hipStream_t stream) {
  pod_status_t st = check_tensors(pl, t);
  if (st != POD_OK) return st;
  if (!pl->has_bp)
    return set_err(POD_ERR_INVALID_ARGUMENT, "plan was made without POD_FLAG_BATCHED_PREFILL");
  const WorkLists& w = pl->bp;
  KernelArgs a = make_args(pl, t, w, pl->dl_bp);
  pick_counters(pl, kKindSeq, stream, &a);
  if (w.n_p() > 0) {
    hipError_t e = launch_prefill(a, kv_mode_of(pl), w.n_p(), stream, /*batched=*/true);
    if (e != hipSuccess) return hip_err(e, "batched prefill kernel launch");
    if (!a.self_reset) ++pl->launches[kKindSeq];
  }
  return launch_merge_of(a, w, stream);
}

pod_status_t pod_attn_merge(const float* part_o, const float* part_lse, int32_t n_rows,
                            int32_t n_splits, void* o, float* lse, hipStream_t stream) {
  if (n_rows < 0 || n_splits < 1 || n_splits > kMaxMergeSplits)
    return set_err(POD_ERR_INVALID_ARGUMENT, "n_rows must be >= 0 and n_splits in [1, 64]");
  if ((int64_t)n_rows * n_splits > (int64_t)INT32_MAX)
    return set_err(POD_ERR_UNSUPPORTED, "too many partials");
  if (n_rows == 0) return POD_OK;
  if (!part_o || !part_lse || !o)
    return set_err(POD_ERR_INVALID_ARGUMENT, "part_o, part_lse or o is NULL");
  if (!aligned16(part_o) || !aligned16(o))
    return set_err(POD_ERR_INVALID_ARGUMENT, "part_o and o must be 16-byte aligned");
  KernelArgs a;
  std::memset(&a, 0, sizeof(a));
  a.part_o = const_cast<float*>(part_o);
  a.part_lse = const_cast<float*>(part_lse);
  a.o_prefill = (uint16_t*)o;
  a.lse_prefill = lse;
  a.m_tasks = nullptr;
  a.n_m = n_rows;
  a.merge_splits = n_splits;
  a.merge_lse_scale = 1.4426950408889634f;
  hipError_t e = launch_merge(a, (n_rows + kMergeTasksPerWG - 1) / kMergeTasksPerWG, stream);
  return e == hipSuccess ? POD_OK : hip_err(e, "merge kernel launch");
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
  out->one_unit_per_wg = pl->choice.one_unit ? 1 : 0;
  out->num_partials = pl->n_partials;
  out->trace_records = pl->trace_records;
  out->runs_sequential = pl->choice.runs_sequential;
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
    case 8: v = &pl->bp.p_items; break;
    case 9: v = &pl->bp.m_tasks; break;
    case 10: v = &pl->bp.pool_off; break;
    case 11: v = &pl->members; break;
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

pod_status_t pod_attn_probe_read_bw(const void* buf, size_t bytes, uint32_t* sink,
                                    int32_t num_blocks, hipStream_t stream) {
  if (!buf || !sink || num_blocks < 1 || bytes < 16 || !aligned16(buf))
    return set_err(POD_ERR_INVALID_ARGUMENT, "bad read-probe arguments");
  hipError_t e = launch_read_probe(buf, (int64_t)(bytes / 16), 0x9E3779B9u, sink, num_blocks, stream);
  return e == hipSuccess ? POD_OK : hip_err(e, "read-probe kernel launch");
}

}  // extern "C"
