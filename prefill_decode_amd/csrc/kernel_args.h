// Arguments of the HIP kernels (passed by value) and their host launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/pod_attn.h"

namespace pod {

constexpr int kMaxPools = 16;

// Counter layout.  A run's claim and completion counters are device-scope
// atomics, which the MI355X serialises per address (about 11 ns each, a few
// hundred ns of latency); each hot counter therefore gets its own 4 KiB so
// that counters of different XCDs proceed in parallel.
constexpr int kCtrStride = 1024;           // ints between two hot counters
constexpr int CS_POOL = 0;                 // +pool: claims from prefill pool (< kMaxPools)
constexpr int CS_DQ = 16;                  // +queue: claims from decode queue (< kMaxPools)
constexpr int CS_DONE = 32;                // +g (8 groups by blockIdx % 8): finished WGs
constexpr int CS_DONE_ALL = 40;            // groups whose WGs all finished
constexpr int kCtrSlots = 41;
constexpr int kCtrBlockInts = kCtrSlots * kCtrStride;
constexpr int kFusedBlock = 0;             // fused kernel's counter block
constexpr int kSeqBlock = kCtrBlockInts;   // sequential prefill kernel's block
constexpr int kCuCounterOff = 2 * kCtrBlockInts;
constexpr int kCuCounters = 2048;          // per-CU role counters (fused kernel)
constexpr int kCounterInts = kCuCounterOff + kCuCounters;

// KV addressing modes (kernel template parameter).
enum KvMode : int { KV_CONTIG = 0, KV_PAGED_WIDE = 1, KV_PAGED_NARROW = 2 };

struct KernelArgs {
  const uint16_t* q_prefill;
  const uint16_t* q_decode;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_indptr;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  uint16_t* o_prefill;
  uint16_t* o_decode;
  float* lse_prefill;
  float* lse_decode;
  float* part_o;          // [n_partials, 128] fp32
  float* part_lse;        // [n_partials] fp32, log2 domain
  const int32_t* p_items;
  const int32_t* d_items;
  const int32_t* m_tasks;
  int32_t* counters;      // the launch's counter block (fused or sequential)
  int32_t* cu_counters;   // per-CU counters (fused)
  int32_t n_dq;           // decode queues (one per XCD): queue q holds units q, q+n_dq, ..
  pod_trace_record_t* trace;
  int32_t n_p, n_d, n_groups, n_m;
  int32_t num_pools;
  int32_t pool_off[kMaxPools + 1];
  int32_t hq, hkv, group;
  int32_t p_heads;        // query heads per prefill item (prefill_heads(group))
  int32_t page_shift;     // log2(page_size) when paged
  int32_t causal;
  float scale_log2;       // sm_scale * log2(e)
  int32_t wgs_per_cu, prefill_quarters, sched_mode;
};

hipError_t launch_fused(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_prefill(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_decode(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_merge(const KernelArgs& a, int grid, hipStream_t s);
hipError_t launch_probe(int32_t* out, int blocks, hipStream_t s);

}  // namespace pod
