// Host planner for one hybrid batch: work lists, KV splits, prefill:decode
// mix.  Pure C++ (no HIP), so it can be tested and sanitised on a CPU.
//
// Sources: [POD] "POD-Attention: Unlocking Full Prefill-Decode Overlap for
// Faster LLM Inference", section "How POD-Attention overlaps" (remapped
// work identities, per-SM role tickets, 2 or 4 blocks per SM, KV splits
// capped at two waves) and "The idea" (proportional, not 50:50, allocation);
// [PR] "Limit kv split when prefill tokens <= 1536" (split count of small
// prefills accounts for co-located decode workgroups).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pod_attn.h"

namespace pod {

// Tile shapes shared by planner and kernels.
constexpr int kHeadDim = 128;
constexpr int kPrefillRows = 256;   // (position, head) rows per prefill item (4 waves x 64)
constexpr int kWaveRows = 64;       // rows per wave: two 32-row MFMA blocks
constexpr int kPrefillKeys = 64;    // keys per prefill KV tile
constexpr int kDecodeStep = 32;     // keys per decode step (2 MFMA key blocks)
constexpr int kDecodeRows = 16;     // decode query tile (MFMA 16 rows)
constexpr int kWavesPerWG = 4;
constexpr int kMaxXcds = 16;
constexpr int kMaxPrefillSplits = 16;
constexpr int kMaxDecodeSplits = 64;
constexpr int kMaxMergeSplits = 64;     // partials one merge task combines
constexpr int kMergeTasksPerWG = 16;    // merge: 4 tasks per wavefront (16 lanes each)
constexpr int kMinDecodeChunk = 512;   // keys per decode split, lower bound
// ... and the bound when the decode keys cannot give every decode wavefront
// a unit of kMinDecodeChunk keys: a wave streams a unit at the rate its own
// loads in flight allow, so small batches need short units to use the GPU
// (the tiny batch: 41.7 -> 29.3 us fused, 41.8 -> 27.2 us sequential)
constexpr int kMinDecodeChunkSmall = 128;
constexpr int kFusedDecodeUnitsPerWave = 2;   // decode units per decode wavefront slot
constexpr int kSeqDecodeUnitsPerWave = 2;
// prefill KV splits aim at this many half-items per prefill slot (the split
// count is rounded down): more items shorten the tail, fewer write and merge
// fewer partials.  The fused plan takes 1.5 items per slot of the prefill CUs
// when the prefill is small (<= 1536 tokens: the decode forms the launch's
// tail, and the prefill need only finish beside it) and 3 per slot of the
// whole GPU when it is large (its last items form the tail, and finer items
// balance it).  Measured in interleaved runs: 1.5 against 2 per slot, 3.5%
// faster on the llama3-8b layer; 3 against 2, 5% faster on the 70B layer
// (against 1 or 4: 1%; the batched mix and the llama2-7b layer keep their
// speed).  The sequential plan takes one item per slot.
constexpr int kFusedPrefillHalfItemsPerSlotSmall = 3;
constexpr int kFusedPrefillHalfItemsPerSlotLarge = 6;
constexpr int kSeqPrefillHalfItemsPerSlot = 2;

// Prefill work item (8 int32).
enum PItem : int {
  P_QROW0 = 0,    // global row of q_prefill holding the item's first position
  P_HEAD = 1,     // first query head; the item covers prefill_heads(g) heads
  P_NROWS = 2,    // valid positions, 1..kPrefillRows / prefill_heads(g)
  P_POS0 = 3,     // absolute position of the first row (kv_len - qo_len + row)
  P_KV_BEGIN = 4, // first key of this split (multiple of kPrefillKeys)
  P_KV_END = 5,   // one past the last key this split may read
  P_KVREQ = 6,    // request index into kv_indptr / page_indptr
  P_PART = 7,     // -1: write O/LSE; else partial index of row 0, where the
                  // row of (head slot j, position i) is j * positions + i
  P_FIELDS = 8
};

// Decode work item (8 int32): one wavefront's unit.
enum DItem : int {
  D_QROW = 0,     // decode request index (row of q_decode)
  D_HEAD0 = 1,    // first query head of the unit (all share one KV head)
  D_NQ = 2,       // query heads, 1..kDecodeRows
  D_KV_BEGIN = 3, // first key (multiple of kDecodeStep)
  D_KV_END = 4,   // one past the last key
  D_KVREQ = 5,    // request index into kv_indptr / page_indptr
  D_PART = 6,     // -1: write O/LSE; else partial index of head D_HEAD0
  D_PSTRIDE = 7,  // partial index step between consecutive heads
  D_FIELDS = 8
};

// Merge task (4 int32): one (row, head) combined from n partials.
enum MTask : int {
  M_OUT = 0,      // row * Hq + head in o_prefill/o_decode (elements of 128)
  M_BASE = 1,     // partial index of split 0
  M_STRIDE = 2,   // partial index step between splits
  M_NFLAG = 3,    // n_splits | (is_decode << 16)
  M_FIELDS = 4
};

// Query heads packed into one prefill item (they share one KV head, so one
// staged K/V tile serves all of them): 4, 2 or 1, the largest dividing the
// group size Hq / Hkv.
inline int32_t prefill_heads(int32_t group) {
  return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}
// positions per prefill item
inline int32_t prefill_positions(int32_t group) { return kPrefillRows / prefill_heads(group); }

struct WorkLists {
  std::vector<int32_t> p_items;    // P_FIELDS each, grouped by XCD pool
  std::vector<int32_t> pool_off;   // num_xcds + 1 offsets (items) into p_items
  std::vector<int32_t> d_items;    // D_FIELDS each, in groups of kWavesPerWG
  std::vector<int32_t> m_tasks;    // M_FIELDS each
  int32_t n_partials = 0;
  int32_t p_splits_max = 1;
  int32_t d_splits_max = 1;
  int32_t n_p() const { return (int32_t)(p_items.size() / P_FIELDS); }
  int32_t n_d() const { return (int32_t)(d_items.size() / D_FIELDS); }
  int32_t n_groups() const { return (n_d() + kWavesPerWG - 1) / kWavesPerWG; }
  int32_t n_m() const { return (int32_t)(m_tasks.size() / M_FIELDS); }
};

struct Batch {
  pod_attn_params_t params;
  std::vector<int32_t> qo, pkv, dkv;   // prefill qo/kv, decode kv
};

struct PlanChoice {
  int32_t wgs_per_cu = 2;
  int32_t prefill_quarters = 4;        // target prefill WGs per CU, in quarters
  int32_t sched_mode = POD_SCHED_SPLIT;   // resolved mode (never AUTO)
};

// Validation of parameters and lengths; returns POD_OK or an error with text.
pod_status_t validate(const pod_attn_params_t* p, int32_t np, const int32_t* qo,
                      const int32_t* pkv, int32_t nd, const int32_t* dkv,
                      const pod_attn_tuning_t* t, std::string* err);

// Proportional prefill share ([POD] "The idea"): quarters of a CU's
// workgroup slots (COLOCATE) or eighths of the CUs (SPLIT) given to prefill,
// from estimated prefill and decode times.
int32_t auto_prefill_quarters(const Batch& b, int32_t wgs_per_cu, int32_t sched_mode);

// Builds one set of work lists.  `prefill_slots` / `decode_wave_slots` are the
// concurrent prefill workgroups / decode wavefronts the splits should fill
// (prefill: about `p_half_items_per_slot` / 2 items per slot);
// decode requests are split until there are about `d_units_per_slot` units
// per decode wavefront (chunks of at least kMinDecodeChunk keys, or
// kMinDecodeChunkSmall when the batch has too few decode keys for that).
void build_lists(const Batch& b, const pod_device_desc_t& dev,
                 int64_t prefill_slots, int32_t p_half_items_per_slot, int64_t decode_wave_slots,
                 int32_t d_units_per_slot, int32_t force_p_splits, int32_t force_d_splits,
                 WorkLists* out);

}  // namespace pod
