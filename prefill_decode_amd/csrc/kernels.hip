// HIP kernels (gfx950 / CDNA4) for fused prefill+decode attention.
//
// Sources: [POD] "POD-Attention: Unlocking Full Prefill-Decode Overlap for
// Faster LLM Inference" (summary page), section "How POD-Attention overlaps":
//   - "Fuse prefill and decode attention into one kernel": one launch with
//     (prefill + decode) workgroups whose work identities are remapped;
//   - "Self-assign roles per SM in software": a leader reads the hardware
//     placement register and takes a per-CU counter value that decides the
//     role;
//   - "Shrink decode tiles to free the tensor cores": decode query tile 16;
//   - "Balance shared memory and threadblock count": decode workgroups are
//     split into single-wave virtual blocks with no workgroup barrier;
//   - "Cap prefill splitting to avoid contention": KV splits (FlashDecoding
//     style) whose partials are merged by log-sum-exp ([PAT] abstract).
//
// Design for gfx950 (not a translation of the pages' CUDA kernels):
//   prefill  128 query rows x 1 head per workgroup (4 waves x 32 rows), keys
//            in tiles of 64 staged through LDS (double buffered; V stored
//            transposed), S^T = K Q^T and O^T += V^T P^T on
//            v_mfma_f32_32x32x16_bf16 so that each lane owns one query row:
//            the softmax state is lane-local and P feeds the next MFMA
//            straight from the accumulator registers.
//   decode   one wavefront = one unit (request, KV head, <=16 query heads,
//            KV split); K is loaded from HBM directly in MFMA operand layout
//            (16-byte loads), V is loaded as full 256-byte rows and transposed
//            through a per-wave LDS slice; 16x16x32 MFMAs; loads of step i+1
//            are in flight while step i computes.
//   merge    one wavefront per (row, head): log-sum-exp of split partials.
// All softmax arithmetic is fp32 in the log2 domain (scores scaled by
// sm_scale*log2(e), exp2); LSE is converted to natural log on output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernel_args.h"
#include "plan.h"

namespace pod {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// LDS geometry (elements of 16 bits).
constexpr int kKStr = kHeadDim + 8;          // prefill K tile row: 64 keys x 136
constexpr int kVtStr = kPrefillKeys + 4;     // prefill V^T tile row: 128 d x 68
constexpr int kKTileElems = kPrefillKeys * kKStr;
constexpr int kVtTileElems = kHeadDim * kVtStr;
constexpr int kPrefillBufElems = kKTileElems + kVtTileElems;
constexpr int kPrefillLdsBytes = 2 * kPrefillBufElems * 2;          // 69632
constexpr int kDecVtStr = kDecodeStep + 8;   // decode V^T slice row: 128 d x 40
constexpr int kDecWaveElems = kHeadDim * kDecVtStr;
constexpr int kDecodeLdsBytes = kWavesPerWG * kDecWaveElems * 2;    // 40960
constexpr int kFusedLdsBytes =
    kPrefillLdsBytes > kDecodeLdsBytes ? kPrefillLdsBytes : kDecodeLdsBytes;

__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float fmax_(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float xor_shfl(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ void lds_fence() {
  // LDS accesses of one wavefront execute in order; this keeps the compiler
  // from moving LDS reads above the writes of other lanes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
// low 16-bit halves of (a, b) -> (a.lo | b.lo << 16); high halves likewise
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---------------------------------------------------------------------------
// KV addressing: token -> row index in units of Hkv*128 elements.
// ---------------------------------------------------------------------------
template <int KVM>
struct KvAddr {
  const int32_t* pages;   // page_indices + page_indptr[req] (paged)
  int64_t base;           // kv_indptr[req] (contiguous)
  int shift;
  __device__ __forceinline__ void init(const KernelArgs& a, int kvreq) {
    if (KVM == KV_CONTIG) {
      base = a.kv_indptr[kvreq];
      pages = nullptr;
    } else {
      base = 0;
      pages = a.page_indices + a.page_indptr[kvreq];
    }
    shift = a.page_shift;
  }
  // generic per-lane lookup (any page size)
  __device__ __forceinline__ int64_t row(int t) const {
    if (KVM == KV_CONTIG) return base + t;
    const int pg = pages[t >> shift];
    return ((int64_t)pg << shift) + (t & ((1 << shift) - 1));
  }
  // row of token t0 + i where [t0, t0 + 16) is 16-aligned and lies in one
  // page (page_size >= 16); `pg` is that page's index (uniform)
  __device__ __forceinline__ int64_t row_in(int pg, int t0, int i) const {
    return ((int64_t)pg << shift) + (t0 & ((1 << shift) - 1)) + i;
  }
};

// ---------------------------------------------------------------------------
// Prefill: 128 query rows x one head over keys [kv_begin, kv_end).
// ---------------------------------------------------------------------------
template <int KVM>
__device__ __forceinline__ void prefill_tile(const KernelArgs& a, const int32_t* it,
                                             uint16_t* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5;            // half of the wave
  const int l32 = lane & 31;
  const int qrow0 = rfl(it[P_QROW0]), head = rfl(it[P_HEAD]), nrows = rfl(it[P_NROWS]);
  const int pos0 = rfl(it[P_POS0]), kv_begin = rfl(it[P_KV_BEGIN]), kv_end = rfl(it[P_KV_END]);
  const int kvreq = rfl(it[P_KVREQ]), part = rfl(it[P_PART]);
  const int kvh = head / a.group;
  const int64_t tok_stride = (int64_t)a.hkv * kHeadDim;
  const uint16_t* kg = a.k + kvh * kHeadDim;
  const uint16_t* vg = a.v + kvh * kHeadDim;
  KvAddr<KVM> addr;
  addr.init(a, kvreq);

  // Q^T operand: lane holds row (wave*32 + l32), d = 16*kk + 8*hl + e
  const int row = wave * 32 + l32;
  const bool row_ok = row < nrows;
  u32x4 qf[8];
  {
    const uint16_t* qp = a.q_prefill +
        ((int64_t)(qrow0 + (row_ok ? row : 0)) * a.hq + head) * kHeadDim + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = row_ok ? *(const u32x4*)(qp + 16 * kk) : u32x4{0, 0, 0, 0};
  }

  // staging assignment: K chunk (key = (tid>>4) + 16 i, d = 8*(tid&15));
  // V quad (keys 4*(tid&15) + i, d = 8*(tid>>4))
  const int kc_key = tid >> 4, kc_d = 8 * (tid & 15);
  const int vq_key = 4 * (tid & 15), vq_d = 8 * (tid >> 4);
  u32x4 kr[4], vr[4];

  auto load_tile = [&](int k0) {
    int pg[4];
    if (KVM == KV_PAGED_WIDE) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int t = k0 + 16 * b;
        pg[b] = t < kv_end ? addr.pages[t >> addr.shift] : 0;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kc_key + 16 * i, t = k0 + key;
      int64_t r;
      if (KVM == KV_PAGED_WIDE) r = addr.row_in(pg[i], k0 + 16 * i, kc_key);
      else r = t < kv_end ? addr.row(t) : 0;
      kr[i] = t < kv_end ? *(const u32x4*)(kg + r * tok_stride + kc_d) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = vq_key + i, t = k0 + key;
      int64_t r;
      if (KVM == KV_PAGED_WIDE) r = addr.row_in(pg[key >> 4], k0 + (key & ~15), key & 15);
      else r = t < kv_end ? addr.row(t) : 0;
      vr[i] = t < kv_end ? *(const u32x4*)(vg + r * tok_stride + vq_d) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](uint16_t* buf) {
    uint16_t* ks = buf;
    uint16_t* vt = buf + kKTileElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(ks + (kc_key + 16 * i) * kKStr + kc_d) = kr[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x2 lo = {lo_halves(vr[0][w], vr[1][w]), lo_halves(vr[2][w], vr[3][w])};
      const u32x2 hi = {hi_halves(vr[0][w], vr[1][w]), hi_halves(vr[2][w], vr[3][w])};
      *(u32x2*)(vt + (vq_d + 2 * w) * kVtStr + vq_key) = lo;
      *(u32x2*)(vt + (vq_d + 2 * w + 1) * kVtStr + vq_key) = hi;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  const int qpos = pos0 + row;                      // this lane's query position
  const int wave_pos_lo = pos0 + wave * 32;         // smallest position of the wave
  const int wave_pos_hi = wave_pos_lo + 31;
  const float sl2 = a.scale_log2;
  const bool causal = a.causal != 0;

  const int ntiles = (kv_end - kv_begin + kPrefillKeys - 1) / kPrefillKeys;
  load_tile(kv_begin);
  store_tile(lds);
  if (ntiles > 1) load_tile(kv_begin + kPrefillKeys);

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    const uint16_t* buf = lds + (t & 1) * kPrefillBufElems;
    if (t + 1 < ntiles) {
      store_tile(lds + ((t + 1) & 1) * kPrefillBufElems);
      if (t + 2 < ntiles) load_tile(kv_begin + (t + 2) * kPrefillKeys);
    }
    const int k0 = kv_begin + t * kPrefillKeys;
    // whole tile in the future of every row of this wave: nothing to do
    if (causal && k0 > wave_pos_hi) continue;
    const uint16_t* ks = buf;
    const uint16_t* vt = buf + kKTileElems;

    // S^T[key][query] for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = 0.0f;
      const uint16_t* kp = ks + (32 * sb + l32) * kKStr + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 kf = *(const u32x4*)(kp + 16 * kk);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(kf), as_bf(qf[kk]), s[sb], 0, 0, 0);
      }
    }
    // mask (only where the tile crosses the split end or the diagonal)
    const bool need_mask = (k0 + kPrefillKeys > kv_end) ||
                           (causal && k0 + kPrefillKeys - 1 > wave_pos_lo);
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[sb][r] * sl2;
        if (need_mask) {
          const int key = k0 + 32 * sb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= kv_end || (causal && key > qpos)) x = kNegInf;
        }
        s[sb][r] = x;
        mx = fmax_(mx, x);
      }
    mx = fmax_(mx, xor_shfl(mx, 32));
    const float m_new = fmax_(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_(m_run - m_use);
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_(s[sb][r] - m_use);
        s[sb][r] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // P^T operands: k-step kk uses block kk>>1, registers 8*(kk&1) .. +7
    u32x4 pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pb[kk][e] = pack_bf16x2(s[kk >> 1][8 * (kk & 1) + 2 * e],
                                s[kk >> 1][8 * (kk & 1) + 2 * e + 1]);
    // O^T[d][query] += V^T[d][key] P^T[key][query]
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint16_t* vrow = vt + (32 * db + l32) * kVtStr + 4 * hl;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ko = 32 * (kk >> 1) + 16 * (kk & 1);
        const u32x2 v0 = *(const u32x2*)(vrow + ko);
        const u32x2 v1 = *(const u32x2*)(vrow + ko + 8);
        const u32x4 af = {v0[0], v0[1], v1[0], v1[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(af), as_bf(pb[kk]), o[db], 0, 0, 0);
      }
    }
  }

  // epilogue: lanes l and l^32 hold the same query row
  const float l_tot = l_run + xor_shfl(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse2 = l_tot > 0.0f ? m_run + log2_(l_tot) : kNegInf;
  if (part < 0) {
    uint16_t* op = a.o_prefill + ((int64_t)(qrow0 + row) * a.hq + head) * kHeadDim + 4 * hl;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                         pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
        *(u32x2*)(op + 32 * db + 8 * g4) = w;
      }
    if (hl == 0 && a.lse_prefill)
      a.lse_prefill[(int64_t)(qrow0 + row) * a.hq + head] = lse2 * kLn2;
  } else {
    const int pi = part + row;
    float* pp = a.part_o + (int64_t)pi * kHeadDim + 4 * hl;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 w = {o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv,
                         o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv};
        *(f32x4*)(pp + 32 * db + 8 * g4) = w;
      }
    if (hl == 0) a.part_lse[pi] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Decode: one wavefront, <=16 query heads sharing a KV head, keys [kb, ke).
// ---------------------------------------------------------------------------
template <int KVM>
__device__ __forceinline__ void decode_unit(const KernelArgs& a, const int32_t* it,
                                            uint16_t* vt) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q4 = lane >> 4;
  const int qi = rfl(it[D_QROW]), h0 = rfl(it[D_HEAD0]), nq = rfl(it[D_NQ]);
  const int kb = rfl(it[D_KV_BEGIN]), ke = rfl(it[D_KV_END]), kvreq = rfl(it[D_KVREQ]);
  const int part = rfl(it[D_PART]), pstride = rfl(it[D_PSTRIDE]);
  const int kvh = h0 / a.group;
  const int64_t tok_stride = (int64_t)a.hkv * kHeadDim;
  const uint16_t* kg = a.k + kvh * kHeadDim;
  const uint16_t* vg = a.v + kvh * kHeadDim;
  KvAddr<KVM> addr;
  addr.init(a, kvreq);

  // Q^T operand: lane holds query j (head h0 + j), d = 32*kk + 8*q4 + e
  u32x4 qf[4];
  {
    const bool ok = j < nq;
    const uint16_t* qp = a.q_decode + ((int64_t)qi * a.hq + h0 + (ok ? j : 0)) * kHeadDim + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = ok ? *(const u32x4*)(qp + 32 * kk) : u32x4{0, 0, 0, 0};
  }

  // K operand: key k0 + 16*sb + j, d = 32*kk + 8*q4 (register sb*4 + kk)
  // V rows:    key k0 + 8*q4 + i, d = 8*j .. 8*j+7     (register i)
  auto load_step = [&](int k0, u32x4 (&kr)[8], u32x4 (&vr)[8]) {
    int64_t krow[2], vrow0 = 0;
    if (KVM == KV_PAGED_WIDE) {
      const int pg0 = addr.pages[k0 >> addr.shift];
      const int pg1 = k0 + 16 < ke ? addr.pages[(k0 + 16) >> addr.shift] : pg0;
      krow[0] = addr.row_in(pg0, k0, j);
      krow[1] = addr.row_in(pg1, k0 + 16, j);
      vrow0 = addr.row_in(q4 < 2 ? pg0 : pg1, k0 + 16 * (q4 >> 1), 8 * (q4 & 1));
    } else if (KVM == KV_CONTIG) {
      krow[0] = addr.base + k0 + j;
      krow[1] = addr.base + k0 + 16 + j;
      vrow0 = addr.base + k0 + 8 * q4;
    } else {
      krow[0] = k0 + j < ke ? addr.row(k0 + j) : 0;
      krow[1] = k0 + 16 + j < ke ? addr.row(k0 + 16 + j) : 0;
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const bool ok = k0 + 16 * sb + j < ke;
      const uint16_t* p = kg + krow[sb] * tok_stride + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kr[sb * 4 + kk] = ok ? *(const u32x4*)(p + 32 * kk) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = k0 + 8 * q4 + i;
      int64_t r;
      if (KVM == KV_PAGED_NARROW) r = t < ke ? addr.row(t) : 0;
      else r = vrow0 + i;
      vr[i] = t < ke ? *(const u32x4*)(vg + r * tok_stride + 8 * j) : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf, l_run = 0.0f;
  const float sl2 = a.scale_log2;

  auto compute_step = [&](int k0, const u32x4 (&kr)[8], const u32x4 (&vr)[8]) {
    f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kr[kk]), as_bf(qf[kk]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kr[4 + kk]), as_bf(qf[kk]), s1, 0, 0, 0);
    }
    // s0[r]: key k0 + 4*q4 + r; s1[r]: key k0 + 16 + 4*q4 + r; query j
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r] * sl2;
      x[4 + r] = s1[r] * sl2;
    }
    if (k0 + kDecodeStep > ke) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + 4 * q4 + r >= ke) x[r] = kNegInf;
        if (k0 + 16 + 4 * q4 + r >= ke) x[4 + r] = kNegInf;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmax_(mx, x[r]);
    mx = fmax_(mx, xor_shfl(mx, 16));
    mx = fmax_(mx, xor_shfl(mx, 32));
    const float m_new = fmax_(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = exp2_(m_run - m_use);
    m_run = m_new;
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x[r] = exp2_(x[r] - m_use);
      ls += x[r];
    }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;

    // V^T slice: row d = 8*j + 2*w (+1), keys 8*q4 .. 8*q4+7
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4 lo = {lo_halves(vr[0][w], vr[1][w]), lo_halves(vr[2][w], vr[3][w]),
                        lo_halves(vr[4][w], vr[5][w]), lo_halves(vr[6][w], vr[7][w])};
      const u32x4 hi = {hi_halves(vr[0][w], vr[1][w]), hi_halves(vr[2][w], vr[3][w]),
                        hi_halves(vr[4][w], vr[5][w]), hi_halves(vr[6][w], vr[7][w])};
      *(u32x4*)(vt + (8 * j + 2 * w) * kDecVtStr + 8 * q4) = lo;
      *(u32x4*)(vt + (8 * j + 2 * w + 1) * kDecVtStr + 8 * q4) = hi;
    }
    lds_fence();
    // P^T operand: e = 0..3 -> key 4*q4 + e, e = 4..7 -> key 16 + 4*q4 + e - 4
    const u32x4 pb = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* vrow = vt + (16 * db + j) * kDecVtStr + 4 * q4;
      const u32x2 v0 = *(const u32x2*)(vrow);
      const u32x2 v1 = *(const u32x2*)(vrow + 16);
      const u32x4 af = {v0[0], v0[1], v1[0], v1[1]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(af), as_bf(pb), o[db], 0, 0, 0);
    }
    lds_fence();
  };

  u32x4 ka[8], va[8], kn[8], vn[8];
  int k0 = kb;
  if (k0 < ke) load_step(k0, ka, va);
  while (k0 < ke) {
    if (k0 + kDecodeStep < ke) load_step(k0 + kDecodeStep, kn, vn);
    compute_step(k0, ka, va);
    k0 += kDecodeStep;
    if (k0 >= ke) break;
    if (k0 + kDecodeStep < ke) load_step(k0 + kDecodeStep, ka, va);
    compute_step(k0, kn, vn);
    k0 += kDecodeStep;
  }

  // epilogue: query j is spread over lanes j, j+16, j+32, j+48
  float l_tot = l_run + xor_shfl(l_run, 16);
  l_tot += xor_shfl(l_tot, 32);
  if (j >= nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse2 = l_tot > 0.0f ? m_run + log2_(l_tot) : kNegInf;
  if (part < 0) {
    uint16_t* op = a.o_decode + ((int64_t)qi * a.hq + h0 + j) * kHeadDim + 4 * q4;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2 w = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                       pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
      *(u32x2*)(op + 16 * db) = w;
    }
    if (q4 == 0 && a.lse_decode) a.lse_decode[(int64_t)qi * a.hq + h0 + j] = lse2 * kLn2;
  } else {
    const int pi = part + j * pstride;
    float* pp = a.part_o + (int64_t)pi * kHeadDim + 4 * q4;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(pp + 16 * db) = o[db] * inv;
    if (q4 == 0) a.part_lse[pi] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Scheduling helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int cu_slot_id() {
  // HW_ID (hwreg 4): CU_ID [11:8], SH_ID [12], SE_ID [15:13]; XCC_ID (hwreg 20) [3:0]
  const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
  const unsigned xcc = __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20);
  const int cu = (hw >> 8) & 0xF, sh = (hw >> 12) & 1, se = (hw >> 13) & 0x7;
  return (int)(((xcc & 7) << 8) | (se << 5) | (sh << 4) | cu);
}

__device__ __forceinline__ int claim_prefill(const KernelArgs& a, int xcc) {
  for (int i = 0; i < a.num_pools; ++i) {
    const int p = (xcc + i) % a.num_pools;
    const int n = a.pool_off[p + 1] - a.pool_off[p];
    if (n <= 0) continue;
    if (__hip_atomic_load(&a.counters[C_POOL + p], __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT) >= n)
      continue;
    const int c = atomicAdd(&a.counters[C_POOL + p], 1);
    if (c < n) return a.pool_off[p] + c;
  }
  return -1;
}

__device__ __forceinline__ int claim_decode(const KernelArgs& a) {
  if (a.n_groups <= 0) return -1;
  if (__hip_atomic_load(&a.counters[C_DEC], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
      a.n_groups)
    return -1;
  const int c = atomicAdd(&a.counters[C_DEC], 1);
  return c < a.n_groups ? c : -1;
}

// Last workgroup of a launch resets the launch's claim counters (and, for the
// ticket scheduler, the per-CU tickets) so the next run starts from zero.
__device__ __forceinline__ void finish_launch(const KernelArgs& a, bool reset_cu,
                                              int* s_last) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int d = atomicAdd(&a.counters[C_DONE], 1);
    *s_last = (d == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (*s_last) {
    __threadfence();
    if (threadIdx.x < 18) a.counters[threadIdx.x] = 0;
    if (reset_cu)
      for (int i = threadIdx.x; i < kCuCounters; i += blockDim.x) a.cu_counters[i] = 0;
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <int KVM>
__global__ __launch_bounds__(256, 2) void pod_fused_kernel(KernelArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int s_info[4];
  if (threadIdx.x == 0) {
    const int slot = cu_slot_id();
    const int xcc = slot >> 8;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    int role;   // 0 prefill, 1 decode
    int* cell = &a.cu_counters[slot];
    const int tp = (a.prefill_quarters + (slot & 3)) >> 2;   // prefill target of this CU
    const int td = a.wgs_per_cu - tp;
    if (a.sched_mode == POD_SCHED_LIVE) {
      int old = __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while (true) {
        const int lp = old & 0xFFFF, ld = old >> 16;
        // take the role whose live count is furthest below its target share
        role = (td <= 0) ? 0 : (tp <= 0) ? 1 : ((lp + 1) * td <= (ld + 1) * tp ? 0 : 1);
        const int nw = old + (role == 0 ? 1 : (1 << 16));
        const int got = atomicCAS(cell, old, nw);
        if (got == old) break;
        old = got;
      }
    } else if (a.sched_mode == POD_SCHED_TICKET) {
      const int t = atomicAdd(cell, 1);
      role = (t % a.wgs_per_cu) < tp ? 0 : 1;
    } else {
      role = 0;
    }
    int unit;
    if (role == 0) {
      unit = claim_prefill(a, xcc);
      if (unit < 0) {
        role = 1;
        unit = claim_decode(a);
        if (a.sched_mode == POD_SCHED_LIVE) atomicAdd(cell, (1 << 16) - 1);
      }
    } else {
      unit = claim_decode(a);
      if (unit < 0) {
        role = 0;
        unit = claim_prefill(a, xcc);
        if (a.sched_mode == POD_SCHED_LIVE) atomicAdd(cell, 1 - (1 << 16));
      }
    }
    s_info[0] = role;
    s_info[1] = unit;
    s_info[2] = slot;
    if (a.trace) {
      pod_trace_record_t* r = a.trace + blockIdx.x;
      r->block = blockIdx.x;
      r->cu_slot = slot;
      r->role = role;
      r->unit = unit;
      r->t_start = t0;
    }
  }
  __syncthreads();
  const int role = s_info[0], unit = s_info[1];
  if (unit >= 0) {
    if (role == 0) {
      prefill_tile<KVM>(a, a.p_items + (int64_t)unit * P_FIELDS, lds);
    } else {
      const int wave = threadIdx.x >> 6;
      const int d = unit * kWavesPerWG + wave;
      if (d < a.n_d)
        decode_unit<KVM>(a, a.d_items + (int64_t)d * D_FIELDS, lds + wave * kDecWaveElems);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.sched_mode == POD_SCHED_LIVE)
      atomicSub(&a.cu_counters[s_info[2]], role == 0 ? 1 : (1 << 16));
    if (a.trace) a.trace[blockIdx.x].t_end = __builtin_amdgcn_s_memrealtime();
  }
  finish_launch(a, a.sched_mode == POD_SCHED_TICKET, &s_info[3]);
}

template <int KVM>
__global__ __launch_bounds__(256, 2) void pod_prefill_kernel(KernelArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int s_info[2];
  if (threadIdx.x == 0) s_info[0] = claim_prefill(a, cu_slot_id() >> 8);
  __syncthreads();
  const int unit = s_info[0];
  if (unit >= 0) prefill_tile<KVM>(a, a.p_items + (int64_t)unit * P_FIELDS, lds);
  finish_launch(a, false, &s_info[1]);
}

template <int KVM>
__global__ __launch_bounds__(256, 2) void pod_decode_kernel(KernelArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int wave = threadIdx.x >> 6;
  const int d = blockIdx.x * kWavesPerWG + wave;
  if (d < a.n_d)
    decode_unit<KVM>(a, a.d_items + (int64_t)d * D_FIELDS, lds + wave * kDecWaveElems);
}

__global__ __launch_bounds__(256) void pod_merge_kernel(KernelArgs a) {
  const int w = blockIdx.x * kWavesPerWG + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= a.n_m) return;
  const int32_t* t = a.m_tasks + (int64_t)w * M_FIELDS;
  const int out = t[M_OUT], base = t[M_BASE], stride = t[M_STRIDE];
  const int n = t[M_NFLAG] & 0xFFFF, is_dec = t[M_NFLAG] >> 16;
  float m = kNegInf;
  for (int s = 0; s < n; ++s) m = fmax_(m, a.part_lse[base + s * stride]);
  float acc0 = 0.0f, acc1 = 0.0f, tot = 0.0f;
  if (m != kNegInf) {
    for (int s = 0; s < n; ++s) {
      const int pi = base + s * stride;
      const float wgt = exp2_(a.part_lse[pi] - m);   // 0 for an empty split
      const float2 v = *(const float2*)(a.part_o + (int64_t)pi * kHeadDim + 2 * lane);
      acc0 += wgt * v.x;
      acc1 += wgt * v.y;
      tot += wgt;
    }
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  uint16_t* o = (is_dec ? a.o_decode : a.o_prefill) + (int64_t)out * kHeadDim + 2 * lane;
  *(uint32_t*)o = pack_bf16x2(acc0 * inv, acc1 * inv);
  float* lse = is_dec ? a.lse_decode : a.lse_prefill;
  if (lane == 0 && lse) lse[out] = tot > 0.0f ? (m + log2_(tot)) * kLn2 : kNegInf;
}

__global__ void pod_probe_kernel(int32_t* out) {
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = (int32_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
    out[2 * blockIdx.x + 1] = (int32_t)__builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
#define POD_DISPATCH(KERNEL, LDS)                                                        \
  switch (kv_mode) {                                                                     \
    case KV_CONTIG:                                                                      \
      hipLaunchKernelGGL(KERNEL<KV_CONTIG>, dim3(grid), dim3(256), LDS, s, a);          \
      break;                                                                             \
    case KV_PAGED_WIDE:                                                                  \
      hipLaunchKernelGGL(KERNEL<KV_PAGED_WIDE>, dim3(grid), dim3(256), LDS, s, a);      \
      break;                                                                             \
    default:                                                                             \
      hipLaunchKernelGGL(KERNEL<KV_PAGED_NARROW>, dim3(grid), dim3(256), LDS, s, a);    \
      break;                                                                             \
  }                                                                                      \
  return hipGetLastError();

static hipError_t g_lds_attr_err = hipSuccess;

static void set_lds_attrs_once() {
  const void* fused[3] = {(const void*)pod_fused_kernel<KV_CONTIG>,
                          (const void*)pod_fused_kernel<KV_PAGED_WIDE>,
                          (const void*)pod_fused_kernel<KV_PAGED_NARROW>};
  const void* pre[3] = {(const void*)pod_prefill_kernel<KV_CONTIG>,
                        (const void*)pod_prefill_kernel<KV_PAGED_WIDE>,
                        (const void*)pod_prefill_kernel<KV_PAGED_NARROW>};
  for (int i = 0; i < 3; ++i) {
    hipError_t e = hipFuncSetAttribute(fused[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kFusedLdsBytes);
    if (e != hipSuccess && g_lds_attr_err == hipSuccess) g_lds_attr_err = e;
    e = hipFuncSetAttribute(pre[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                            kPrefillLdsBytes);
    if (e != hipSuccess && g_lds_attr_err == hipSuccess) g_lds_attr_err = e;
  }
}

// Dynamic LDS above 64 KiB must be enabled per kernel before its first launch.
static hipError_t set_lds_attrs() {
  static std::once_flag once;
  std::call_once(once, set_lds_attrs_once);
  return g_lds_attr_err;
}

hipError_t launch_fused(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  if (hipError_t e = set_lds_attrs(); e != hipSuccess) return e;
  POD_DISPATCH(pod_fused_kernel, kFusedLdsBytes)
}

hipError_t launch_prefill(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  if (hipError_t e = set_lds_attrs(); e != hipSuccess) return e;
  POD_DISPATCH(pod_prefill_kernel, kPrefillLdsBytes)
}

hipError_t launch_decode(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  POD_DISPATCH(pod_decode_kernel, kDecodeLdsBytes)
}

hipError_t launch_merge(const KernelArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(pod_merge_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_probe(int32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(pod_probe_kernel, dim3(blocks), dim3(256), 0, s, out);
  return hipGetLastError();
}

}  // namespace pod
