// Arguments of the HIP kernels (passed by value) and their host launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/pod_attn.h"

namespace pod {

constexpr int kMaxPools = 16;

// Counter layout.  A run's claim counters are device-scope atomics, which
// the MI355X serialises per address (about 11 ns each, a few hundred ns of
// latency); each hot counter therefore gets its own 4 KiB so that counters of
// different XCDs proceed in parallel.
//
// Each kind of launch (fused, sequential prefill) has three blocks: launches
// alternate between blocks 0 and 1 by a host-side launch count, and the first
// workgroup of a launch zeroes the block the next launch will use, so no
// completion counting is needed; block 2 serves launches recorded into a
// graph (whose arguments are frozen), which count completions and let the
// last workgroup reset the block.
constexpr int kCtrStride = 1024;           // ints between two hot counters
constexpr int kMaxDecodeQueues = 32;
constexpr int CS_POOL = 0;                 // +pool: claims from prefill pool (< kMaxPools)
constexpr int CS_DQ = 16;                  // +queue: claims from decode queue (< kMaxDecodeQueues)
constexpr int CS_DONE = 48;                // +g (8 groups by blockIdx % 8): finished WGs
constexpr int CS_DONE_ALL = 56;            // groups whose WGs all finished
constexpr int CS_EMPTY = 57;               // +role (0 prefill, 1 decode): every queue of the role was seen empty
constexpr int kCtrSlots = 59;
constexpr int kCuCounters = 2048;          // per-CU role counters (fused kernel), one per
constexpr int kCellStride = 16;            // 64-byte line each
constexpr int kCuCounterOff = kCtrSlots * kCtrStride;
constexpr int kCtrBlockInts = kCuCounterOff + kCuCounters * kCellStride;
constexpr int kBlocksPerKind = 3;          // parity 0, parity 1, self-resetting
constexpr int kKindFused = 0, kKindSeq = 1;
constexpr int kCounterInts = 2 * kBlocksPerKind * kCtrBlockInts;

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
  float* part_o;          // [n_partials, 128] fp32 (each partial divided by its own l)
  float* part_lse;        // [n_partials] fp32, log2 domain (natural log for a
                          // standalone merge, see merge_lse_scale)
  const int32_t* p_items;
  const int32_t* d_items;
  const int32_t* m_tasks;
  int32_t* counters;      // the launch's counter block (hot counters, then per-CU cells)
  int32_t* counters_next; // block the next launch of this kind uses: zeroed here (or NULL)
  int32_t self_reset;     // 1: count completions, last workgroup resets `counters`
  int32_t n_dq;           // decode queues (4 per XCD): queue q holds groups q, q+n_dq, ..
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
  int32_t one_unit;       // 1: every workgroup runs one unit and exits
  int32_t n_preq;         // prefill requests: items with a larger KV request index are
                          // decode requests run through the prefill tile (batched prefill)
  // standalone merge (m_tasks == NULL): task t combines partials t * merge_splits
  // .. + merge_splits - 1 into row t of o_prefill / lse_prefill
  int32_t merge_splits;
  float merge_lse_scale;  // factor taking part_lse to log2 (1, or log2(e) for natural log)
  const float* k_scale;   // FP8 KV: per-KV-head scales (device fp32 [Hkv])
  const float* v_scale;
  int32_t kv_fp8;         // 1: K and V are FP8 E4M3 (the F8 kernels)
  const int32_t* d_members;  // shared-prefix plans: decode index of each group member
  int32_t pack_rpr;          // shared-prefix plans: tile rows per member (min(g, 16))
};

hipError_t launch_fused(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_prefill(const KernelArgs& a, int kv_mode, int grid, hipStream_t s,
                          bool batched = false);
hipError_t launch_decode(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_decode_fp8(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_decode_pack(const KernelArgs& a, int kv_mode, int grid, hipStream_t s);
hipError_t launch_merge(const KernelArgs& a, int grid, hipStream_t s);
hipError_t launch_probe(int32_t* out, int blocks, hipStream_t s);

// Size of the per-device static scratch (pod_attn_plan_scratch), and its
// device address on `device` (which must be the current device on the first
// call for it).
constexpr size_t kScratchBytes = size_t(128) << 20;
hipError_t scratch_address(int device, void** out);
hipError_t launch_read_probe(const void* buf, int64_t n16, uint32_t never, uint32_t* sink,
                             int blocks, hipStream_t s);

}  // namespace pod
