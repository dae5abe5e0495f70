// Arguments of the HIP kernels (passed by value) and their host launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/pod_attn.h"

namespace pod {

constexpr int kMaxPools = 16;

// Counter block layout (int32 offsets inside a plan's counter region).
constexpr int kCuCounters = 2048;          // per-CU role counters (fused kernel)
constexpr int kFusedBlock = 2048;          // fused: pools, decode, done
constexpr int kSeqBlock = 2048 + 32;       // sequential prefill: pools, done
constexpr int kCounterInts = 4096;
constexpr int C_POOL = 0;                  // +pool: claims taken from prefill pool
constexpr int C_DEC = 16;                  // claims taken from the decode groups
constexpr int C_DONE = 17;                 // workgroups finished

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
  pod_trace_record_t* trace;
  int32_t n_p, n_d, n_groups, n_m;
  int32_t num_pools;
  int32_t pool_off[kMaxPools + 1];
  int32_t hq, hkv, group;
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
