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
//   prefill  256 (position, head) rows per workgroup: up to 4 query heads of
//            one KV head x 256/heads positions, 64 rows per wave as two
//            32-row MFMA blocks; keys in 64-key tiles staged by LDS DMA
//            (double buffered, XOR-swizzled rows), S^T = K Q^T and O^T +=
//            V^T P^T on v_mfma_f32_32x32x16_bf16 so that each lane owns one
//            query row: the softmax state is lane-local and P feeds the next
//            MFMA straight from the accumulator registers.
//   decode   one wavefront = one unit (request, KV head, <=16 query heads,
//            KV split); K is loaded from HBM as whole 128-byte lines into
//            registers and rearranged into MFMA operands by DPP row shifts,
//            V goes by LDS DMA into a per-wave slice and is read back
//            transposed; 16x16x32 MFMAs; loads of step i+1 are in flight
//            while step i computes.
//   merge    one 16-lane group per (row, head): log-sum-exp of split partials.
// All softmax arithmetic is fp32 in the log2 domain (scores scaled by
// sm_scale*log2(e), exp2); LSE is converted to natural log on output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

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

// LDS geometry.  K and V tiles are kept row-major ([key][128 d], 256-byte
// rows) exactly as LDS DMA deposits them; the 16-byte chunks of each row are
// XOR-swizzled with bits of the row index (the DMA source addresses carry the
// swizzle) so that the MFMA-operand reads -- ds_read_b128 for K and the
// transposing ds_read_b64_tr_b16 for V^T -- are free of bank conflicts.
constexpr int kRowBytes = kHeadDim * 2;                      // 256
constexpr int kTileBytes = kPrefillKeys * kRowBytes;         // 16384
constexpr int kDecStepBytes = kDecodeStep * kRowBytes;       // 8192
constexpr int kRow8 = kHeadDim;                              // FP8 row: 128 bytes
constexpr int kTile8 = kPrefillKeys * kRow8;                 // 8192
// A workgroup owns two LDS objects of 32 KiB (64 KiB in all, so two
// workgroups fit a CU's 160 KiB): X = {K tile 0, V tile 0}, Y = {K tile 1,
// V tile 1}.  Prefill iteration t reads the tiles of parity t & 1 while the
// DMAs fill the other parity, so it reads one object and fills the other;
// decode wave w keeps its step buffers of parity 0 / 1 at X + 8w KiB / Y +
// 8w KiB.  Because the buffers being filled and the buffers being read are
// distinct objects, the compiler can prove that an LDS DMA in flight does
// not alias the reads and adds no wait for it.
constexpr uint32_t kVSwz = 0xC862EA40u;   // V chunk swizzle by row & 7 (nibble table)

typedef const __attribute__((address_space(4))) int32_t* cptr;   // read-only, scalar-loadable
typedef __attribute__((address_space(3))) void* lds_vptr;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (int)((kVSwz >> (4 * (r & 7))) & 15u); }

__device__ __forceinline__ bf16x8 as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 as_f16(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float fmax_(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }
// value combined with the same lane of the other 32-lane half (v_permlane32_swap)
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// ... and with the other 16-lane row of each 32-lane half (v_permlane16_swap)
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ bool any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
// Compiler-only barrier for one wavefront's LDS traffic.  The hardware keeps
// one wave's LDS instructions in order and s_waitcnt covers LDS DMA, so no
// machine wait is needed; a memory fence here would also wait for the LDS DMA
// of the next step, which is still meant to be in flight.
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }
// s_waitcnt vmcnt(N): this wave's vector-memory operations (loads and LDS
// DMA) issued before the last N have completed.  gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]; the other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Buffer resource over a uniform base (raw, 32-bit byte offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF,
                                           0x00020000);
}
// The same over `bytes` bytes: a load at a larger offset returns zeros (and
// an LDS DMA deposits them) instead of reading memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// cache policy bits of buffer loads: 0 = default, kStream = non-temporal
// (data read once, e.g. a decode request's KV, should not displace reused lines)
constexpr int kStream = 2;
template <int CP = 0>
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP));
}
__device__ __forceinline__ u32x4 gload(const char* p) { return *(const u32x4*)p; }
// LDS DMA: lane L's 16 bytes at base + voff + soff land at lds_dst + 16 L
// (lds_dst uniform across the wave)
template <int CP = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)lds_dst, 16, voff, soff, 0, CP);
}
// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
// (i & 3) of the 4-element reads of lanes 4e + (i >> 2), e = 0..3; with lane x
// reading row k0 + (x >> 2), columns c0 + 4 (x & 3) .. +3 of a row-major
// [k][c] tile, lane i gets column c0 + i of rows k0 .. k0 + 3.
__device__ __forceinline__ u32x2 tr_read(const char* p) {
  const v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<char*>(p)));
  return __builtin_bit_cast(u32x2, t);
}

// eight E4M3 bytes (two dwords, byte order = element order) to eight bf16
// (exact: E4M3 values are bf16 values)
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
#define POD_CVT(w, upper) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, upper))
  return u32x4{POD_CVT(lo, false), POD_CVT(lo, true), POD_CVT(hi, false), POD_CVT(hi, true)};
#undef POD_CVT
}
// the same to eight fp16 (exact: E4M3 values are fp16 values)
__device__ __forceinline__ u32x4 fp8x8_to_f16(uint32_t lo, uint32_t hi) {
#define POD_CVT(w, upper) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, upper))
  return u32x4{POD_CVT(lo, false), POD_CVT(lo, true), POD_CVT(hi, false), POD_CVT(hi, true)};
#undef POD_CVT
}

// ---------------------------------------------------------------------------
// KV addressing: token -> row index in units of Hkv*128 elements.
// ---------------------------------------------------------------------------
template <int KVM>
struct KvAddr {
  cptr pages;             // page_indices + page_indptr[req] (paged)
  int64_t base;           // kv_indptr[req] (contiguous)
  int shift;
  __device__ __forceinline__ void init(const KernelArgs& a, int kvreq) {
    if (KVM == KV_CONTIG) {
      base = ((cptr)a.kv_indptr)[kvreq];
      pages = nullptr;
    } else {
      base = 0;
      pages = (cptr)a.page_indices + ((cptr)a.page_indptr)[kvreq];
    }
    shift = a.page_shift;
  }
  // row of the first token of a 16-key block [t0, t0 + 16) that lies in one
  // page (page_size >= 16) or in the contiguous layout; uniform (scalar)
  __device__ __forceinline__ int64_t block_row(int t0) const {
    if (KVM == KV_CONTIG) return base + t0;
    const int pg = pages[t0 >> shift];
    return ((int64_t)pg << shift) + (t0 & ((1 << shift) - 1));
  }
  // generic per-lane row of token t
  __device__ __forceinline__ int64_t row(int t) const {
    if (KVM == KV_CONTIG) return base + t;
    const int pg = pages[t >> shift];
    return ((int64_t)pg << shift) + (t & ((1 << shift) - 1));
  }
};

// ---------------------------------------------------------------------------
// Prefill item: positions pos0 .. pos0 + nrows - 1 of one request (q rows
// qrow0 + i) for nh query heads head0 .. head0 + nh - 1 that share one KV
// head, over keys [kv_begin, kv_end); 256 (position, head) rows in all.  Wave
// w takes head head0 + w / (4 / nh) and 64 consecutive positions as two
// 32-row MFMA blocks A and B, so that every K and V^T operand read from LDS
// feeds two MFMAs, and one staged K/V tile serves all nh heads.
//
// Keys come in 64-key LDS tiles (double buffered, staged by LDS DMA), each
// processed as two 32-key halves: S^T = K Q^T for blocks A and B (one K
// operand, two MFMAs), the online softmax of both blocks, then O^T += V^T
// P^T (one V^T operand, two MFMAs).  The loop over tiles is unrolled by two
// so that every LDS address is a per-lane base plus an immediate offset.
//
// BP (batched prefill, a comparator of the pages): items whose KV request is
// a decode request (index >= n_preq) read their query row from q_decode and
// write o_decode / lse_decode, i.e. a decode runs through this tile as a
// one-row chunk.
//
// F8 (FP8 E4M3 KV cache, per-KV-head scales): a tile's FP8 K and V rows
// (128 bytes) are staged by LDS DMA into object Y, then the workgroup
// converts them, once for all its waves, into the 16-bit tiles of object X in
// the layout above (K to bf16; V to fp16, exact like bf16), and the halves
// run on X as for bf16, except that P is rounded to fp16 and PV is an fp16
// MFMA: two more mantissa bits for P at the same rate.  The next tile's DMA
// is issued after the conversion (so it never waits on the reads of Y) and
// lands while X is computed.  The K scale multiplies the score with sm_scale,
// the V scale the output.
// ---------------------------------------------------------------------------
template <int KVM, bool BP = false, bool F8 = false>
__device__ __forceinline__ void prefill_tile(const KernelArgs& a, cptr it, char* __restrict__ kt0,
                                             char* __restrict__ kt1, char* __restrict__ vt0,
                                             char* __restrict__ vt1) {
  // The thread index passes through an empty asm so that nothing derived
  // from it is hoisted out of a caller's work loop and kept live across it.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = rfl(tid >> 6);
  const int hl = lane >> 5;            // half of the wave
  const int l32 = lane & 31;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int qrow0 = it[P_QROW0], head0 = it[P_HEAD], nrows = it[P_NROWS];
  const int pos0 = it[P_POS0], kv_begin = it[P_KV_BEGIN], kv_end = it[P_KV_END];
  const int kvreq = it[P_KVREQ], part = it[P_PART];
  const bool dec_item = BP && kvreq >= a.n_preq;
  const uint16_t* const q_src = dec_item ? a.q_decode : a.q_prefill;
  const int wph = kWavesPerWG / a.p_heads;          // waves per head
  const int hidx = wave / wph;
  const int wpos = kWaveRows * (wave - hidx * wph);  // first position (item-relative)
  const int head = head0 + hidx;
  const int kvh = head0 / a.group;
  constexpr int kSrcRow = F8 ? kRow8 : kRowBytes;     // bytes of one head's K or V row
  const uint32_t tok = (uint32_t)a.hkv * kSrcRow;
  const char* kbase = (const char*)a.k + kvh * kSrcRow;
  const char* vbase = (const char*)a.v + kvh * kSrcRow;
  KvAddr<KVM> addr;
  addr.init(a, kvreq);
  const int span = kv_end - kv_begin;
  const int ntiles = (span + kPrefillKeys - 1) / kPrefillKeys;
  const int nfull = span / kPrefillKeys;
  const bool causal = a.causal != 0;
  // FP8: the KV head's scales (uniform, through the scalar cache)
  const float sl2 = F8 ? a.scale_log2 * __builtin_bit_cast(float, ((cptr)a.k_scale)[kvh])
                       : a.scale_log2;
  const float vsc = F8 ? __builtin_bit_cast(float, ((cptr)a.v_scale)[kvh]) : 1.0f;
  // keys this wave needs: tiles [0, t_act); tiles >= t_mask need masking
  const int nvalid = min(kWaveRows, nrows - wpos);  // may be <= 0
  const int pos_lo = pos0 + wpos;
  const int pos_hi = pos_lo + max(nvalid, 1) - 1;
  const int x_act = pos_hi - kv_begin;
  const int t_act = nvalid <= 0 ? 0
                    : !causal    ? ntiles
                    : x_act < 0  ? 0
                                 : min(ntiles, x_act / kPrefillKeys + 1);
  const int t_mask = causal ? min(nfull, max(0, (pos_lo - kv_begin + 1) / kPrefillKeys)) : nfull;

  // Q^T operands of blocks A (positions wpos + l32) and B (+32):
  // lane holds d = 16 kk + 8 hl + e
  const int rA = wpos + l32, rB = rA + 32;          // item-relative positions
  const bool okA = rA < nrows, okB = rB < nrows;
  u32x4 qa[8], qb[8];
  {
    const uint16_t* qpa = q_src +
        ((int64_t)(qrow0 + (okA ? rA : 0)) * a.hq + head) * kHeadDim + 8 * hl;
    const uint16_t* qpb = q_src +
        ((int64_t)(qrow0 + (okB ? rB : 0)) * a.hq + head) * kHeadDim + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qa[kk] = okA ? *(const u32x4*)(qpa + 16 * kk) : u32x4{0, 0, 0, 0};
      qb[kk] = okB ? *(const u32x4*)(qpb + 16 * kk) : u32x4{0, 0, 0, 0};
    }
  }

  // staging: wave w fills rows [16w, 16w + 16) of a tile, four rows per
  // instruction; lane L deposits row 4i + L/16, chunk position L%16, which
  // holds source chunk (L%16) ^ swizzle(row)
  const int wrow = 16 * wave * kRowBytes;           // this wave's rows in a tile
  // A tile's 16-key blocks each lie in one page (page_size >= 16); in the
  // last, partial tile the blocks and the lanes' rows are clamped to the last
  // key (finite data, never read past it).
  const int lastb = (kv_end - 1) & ~15;             // start of the block holding key kv_end-1
  auto bstart = [&](int t) { return min(kv_begin + t * kPrefillKeys + 16 * wave, lastb); };
  auto stage = [&](int t, bool is_k, int buf, __amdgpu_buffer_rsrc_t r) {
    // lane-derived offsets are recomputed here rather than held across the
    // tile loop (registers are the limit of this kernel)
    int sl = threadIdx.x;
    asm volatile("" : "+v"(sl));
    const int dq = (sl >> 4) & 3, dc = sl & 15, lane = sl & 63;
    char* dst = (is_k ? (buf ? kt1 : kt0) : (buf ? vt1 : vt0)) + wrow;
    if (KVM != KV_PAGED_NARROW) {
      const int rmax = kv_end - 1 - bstart(t);
      if (rmax >= 15) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * i + dq;
          const uint32_t vo = dq * tok + 16u * (dc ^ (is_k ? kswz(rr) : vswz(rr)));
          dma16(r, dst + 4 * i * kRowBytes, vo, 4 * i * tok);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * i + dq;
          const uint32_t vo = (uint32_t)min(rr, rmax) * tok +
                              16u * (dc ^ (is_k ? kswz(rr) : vswz(rr)));
          dma16(r, dst + 4 * i * kRowBytes, vo, 0);
        }
      }
    } else {
      const char* gbase = is_k ? kbase : vbase;
      const int k0 = kv_begin + t * kPrefillKeys + 16 * wave;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rt = 16 * wave + 4 * i + dq;                // row in the tile
        const int key = min(k0 + 4 * i + dq, kv_end - 1);     // clamp: finite, never read past
        const int c = dc ^ (is_k ? kswz(rt) : vswz(rt));
        *(u32x4*)(dst + 4 * i * kRowBytes + 16 * lane) =
            gload(gbase + addr.row(key) * tok + 16 * c);
      }
    }
  };
  // resource of this wave's (clamped) 16-key block of tile t, bounded to
  // the block's keys up to kv_end - 1: rows past them read as zeros
  auto block_rsrc = [&](int t, const char* gbase) {
    const int b0 = bstart(t);
    return rsrc_n(gbase + (KVM != KV_PAGED_NARROW ? addr.block_row(b0) : 0) * tok,
                  min(kv_end - b0, 16) * (int)tok);
  };

  // per-lane LDS read offsets (bytes from a tile's base); the half h and
  // the buffer are immediates.  K: row 32 h + l32, chunk (2 kk + hl) ^ swz =
  // 2 (kk ^ (swz >> 1)) + (hl ^ (swz & 1)).
  const int ksw = kswz(l32);
  const uint32_t kofs0 = (uint32_t)(l32 * kRowBytes + 16 * (hl ^ (ksw & 1)));
  const uint32_t kx = (uint32_t)(ksw >> 1);
  // (the per-read offsets are formed from these inside each half; held
  // for the whole loop they would not fit the register file)
  // V^T: rows vrow0 + 32 h + 16 ks (+8), chunk (4 db + c) ^ swz =
  // 4 (db ^ (swz >> 2)) + (c ^ (swz & 3))
  const int vrow0 = 4 * hl + (j16 >> 2);
  const int vsw = vswz(vrow0);
  const uint32_t vofs0 = (uint32_t)(vrow0 * kRowBytes +
                                    16 * ((2 * (g16 & 1) + ((j16 & 3) >> 1)) ^ (vsw & 3)) +
                                    8 * (j16 & 1));
  const uint32_t vx = (uint32_t)(vsw >> 2);


  f32x16 oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    oa[i] = f32x16{};
    ob[i] = f32x16{};
  }
  // Online softmax with a lazy reference max: a row's reference m moves only
  // when the row max exceeds it by more than kLazyLog2, so P = exp2(s - m) <=
  // 2^kLazyLog2 (exact in fp32, one bf16 rounding as any P) and the rescale
  // of O is rare.  O / l are normalised by the same m at the end, so the
  // result is the softmax either way.
  constexpr float kLazyLog2 = 8.0f;
  float ma = kNegInf, la = 0.0f, mb = kNegInf, lb = 0.0f;

  // S^T of one 32-key half for both blocks: one K operand, two MFMAs.  The
  // program order is the issue order: each K operand read one k-step ahead,
  // and after the first MFMA of every odd k-step one DMA of the next tile
  // (dma(i), i = 0..3; a no-op in halves that stage nothing), so a DMA that
  // waits to issue does so while an MFMA runs, and the waves of a CU do not
  // all issue their DMAs at once.
  auto qk = [&](const char* kb, uint32_t k0, uint32_t kxx, f32x16& sa, f32x16& sb, auto dma) {
    auto koff = [&](int kk) { return k0 + 32u * ((uint32_t)kk ^ kxx); };
    sa = f32x16{};
    sb = f32x16{};
    u32x4 kcur = *(const u32x4*)(kb + koff(0));
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 knext = kk < 7 ? *(const u32x4*)(kb + koff(kk + 1)) : kcur;
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(kcur), as_bf(qa[kk]), sa, 0, 0, 0);
      if (kk & 1) dma(kk >> 1);
      sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(kcur), as_bf(qb[kk]), sb, 0, 0, 0);
      kcur = knext;
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (kk < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (kk & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // register r holds key key0 + 8 (r >> 2) + (r & 3) (key0 includes 4 hl);
  // keys below `lim` are visible: r is kept iff its offset < lim - key0
  auto mask = [&](f32x16& sx, int key0, int lim) {
    const int dd = lim - key0;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= dd) sx[r] = kNegInf;
  };
  // row max of a block's S; moves m (and rescales O, l) past the lazy bound
  auto update_max = [&](const f32x16& sx, float& m, float& l, f32x16 (&o)[4]) {
    float mx = sx[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmax_(mx, sx[r]);
    mx = max_x32(mx) * sl2;
    const bool up = mx > m + kLazyLog2;
    if (any_lane(up)) {
      const float m_new = up ? mx : m;
      const float alpha = m_new == kNegInf ? 1.0f : exp2_(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m = m_new;
    }
  };
  // P^T = exp2(S sl2 - m) as two MFMA B operands (k-steps of 16 keys); row
  // sum into l.  k-step ks uses registers 8 ks .. 8 ks + 7.
  auto expsum = [&](f32x16& sx, float m, float& l, u32x4 (&p)[2]) {
    const float nm = m == kNegInf ? 0.0f : -m;
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[r] = exp2_(__builtin_fmaf(sx[r], sl2, nm));
    float ls = sx[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) ls += sx[r];
    l += ls;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[ks][e] = F8 ? pack_f16x2(sx[8 * ks + 2 * e], sx[8 * ks + 2 * e + 1])
                      : pack_bf16x2(sx[8 * ks + 2 * e], sx[8 * ks + 2 * e + 1]);
  };
  // O^T += V^T P^T for one 32-key half: one V^T operand (two transposing
  // reads), two MFMAs; operand reads one ahead and DMAs placed as in qk
  auto pv = [&](const char* vb, uint32_t v0, uint32_t vxx, const u32x4 (&pa)[2],
                const u32x4 (&pb)[2], auto dma) {
    auto vop = [&](int i) {
      const int ks = i >> 2, db = i & 3;
      const char* cp = vb + v0 + 64u * ((uint32_t)db ^ vxx) + 16 * ks * kRowBytes;
      const u32x2 lo = tr_read(cp);
      const u32x2 hi = tr_read(cp + 8 * kRowBytes);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 vcur = vop(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ks = i >> 2, db = i & 3;
      const u32x4 vnext = i < 7 ? vop(i + 1) : vcur;
      if constexpr (F8) {
        oa[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16(vcur), as_f16(pa[ks]), oa[db], 0, 0, 0);
        ob[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16(vcur), as_f16(pb[ks]), ob[db], 0, 0, 0);
      } else {
        oa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(vcur), as_bf(pa[ks]), oa[db], 0, 0, 0);
        if (i & 1) dma(i >> 1);
        ob[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(vcur), as_bf(pb[ks]), ob[db], 0, 0, 0);
      }
      vcur = vnext;
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // one 32-key half h of tile t (buffers K kb, V vb).  No instruction is
  // scheduled across a half's boundaries: overlapping two halves would keep
  // both halves' S and operands live, beyond the register file.
  auto half = [&](int t, int h, const char* kb, const char* vb, bool masked, auto dma_k,
                  auto dma_v) {
    __builtin_amdgcn_sched_barrier(0);
    uint32_t k0 = kofs0, kxx = kx, v0 = vofs0, vxx = vx;
    asm volatile("" : "+v"(k0), "+v"(kxx), "+v"(v0), "+v"(vxx));
    f32x16 sa, sb;
    // MFMA phases run at raised wave priority: on a SIMD shared with another
    // wave in its softmax (VALU) phase, the MFMA issue goes first and the
    // two waves' phases interleave
    __builtin_amdgcn_s_setprio(1);
    qk(kb + 32 * h * kRowBytes, k0, kxx, sa, sb, dma_k);
    __builtin_amdgcn_s_setprio(0);
    if (masked) {
      const int key0 = kv_begin + t * kPrefillKeys + 32 * h + 4 * hl;
      const int qpos = pos0 + wpos + (threadIdx.x & 31);   // block A's row position
      mask(sa, key0, causal ? min(qpos + 1, kv_end) : kv_end);
      mask(sb, key0, causal ? min(qpos + 33, kv_end) : kv_end);
    }
    update_max(sa, ma, la, oa);
    update_max(sb, mb, lb, ob);
    u32x4 pa[2], pb[2];
    expsum(sa, ma, la, pa);
    expsum(sb, mb, lb, pb);
    __builtin_amdgcn_s_setprio(1);
    pv(vb + 32 * h * kRowBytes, v0, vxx, pa, pb, dma_v);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // iteration t: K(t) and V(t) are in LDS buffers t&1; DMA of tile t+1
  // goes to the other buffers, which the barrier released
  __amdgpu_buffer_rsrc_t rk = block_rsrc(0, kbase), rv = block_rsrc(0, vbase);
  if constexpr (!F8) {
    stage(0, true, 0, rk);
    stage(0, false, 0, rv);
  }
  // DMA of row group i (rows 4i .. 4i + 3 of this wave's 16) of tile t into
  // buffers `buf`, without branches, so that it can sit among a half's
  // MFMAs: rows past the last key read as zeros (the block's resource ends
  // there).  Lane L takes row rr = 4i + dq (dq = L/16 % 4) and source chunk
  // dc ^ swz(rr) (dc = L%16).  K's swizzle rr & 15 makes that (dc ^ dq) ^ 4i;
  // V's depends on i only through i & 1 and flips bit 1 with it.  So two
  // lane offsets held across the item give every row group's offset in one
  // VALU (they pass through an empty asm per use, so that the eight
  // derived offsets are not hoisted and held as well).
  const int ldq = (lane >> 4) & 3, ldc = lane & 15;
  const uint32_t dma_k0 = (uint32_t)ldq * tok + 16u * (uint32_t)(ldc ^ ldq);
  const uint32_t dma_v0 = (uint32_t)ldq * tok + 16u * (uint32_t)(ldc ^ vswz(ldq));
  auto dma_row = [&](bool is_k, int buf, __amdgpu_buffer_rsrc_t r, int i) {
    char* dst = (is_k ? (buf ? kt1 : kt0) : (buf ? vt1 : vt0)) + wrow;
    uint32_t b = is_k ? dma_k0 : dma_v0;
    asm volatile("" : "+v"(b));
    const uint32_t vo = (b ^ (is_k ? 64u * i : (i & 1) ? 32u : 0u)) + 4u * i * tok;
    dma16(r, dst + 4 * i * kRowBytes, vo, 0);
  };
  auto nothing = [](int) {};
  auto body = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    wait_vmem<0>();
    __syncthreads();                       // tile t landed; tile t-1's buffers free
    // The next tile goes to the buffers of parity P ^ 1.  With the wide or
    // contiguous layout its DMAs are spread over the first half's MFMAs; the
    // last iteration then restages its own tile there (unread, and waited
    // for before the item ends), which keeps that code free of branches.
    const bool flat = KVM != KV_PAGED_NARROW && t < t_act;
    const int tn = flat ? min(t + 1, ntiles - 1) : t + 1;
    if (tn < ntiles) {
      rk = block_rsrc(tn, kbase);
      rv = block_rsrc(tn, vbase);
      if (!flat) {
        stage(tn, true, P ^ 1, rk);
        stage(tn, false, P ^ 1, rv);
      }
    }
    if (t < t_act) {
      const char* kb = P ? kt1 : kt0;
      const char* vb = P ? vt1 : vt0;
      // the second half is needed unless every key in it is beyond the
      // wave's last position or the KV range
      const int k1 = kv_begin + t * kPrefillKeys + 32;
      const bool h1 = k1 < kv_end && (!causal || k1 <= pos_hi);
      // one copy of the half's code (a masked and an unmasked copy would
      // double the live ranges the register allocator has to cover)
      const bool masked = t >= t_mask;
      if (KVM != KV_PAGED_NARROW)
        half(t, 0, kb, vb, masked, [&](int i) { dma_row(true, P ^ 1, rk, i); },
             [&](int i) { dma_row(false, P ^ 1, rv, i); });
      else
        half(t, 0, kb, vb, masked, nothing, nothing);
      if (h1) half(t, 1, kb, vb, masked, nothing, nothing);
    }
  };
  if constexpr (F8) {
    // stage: this wave's 16 rows of tile t, eight 128-byte rows per DMA
    // (lane L: row L / 8, chunk L % 8), into Y's K and V staging tiles;
    // rows past the last key read as zeros (bounded block resource)
    char* const k8 = kt1;
    char* const v8 = vt1;
    auto stage8 = [&](int t) {
      int sl = threadIdx.x;
      asm volatile("" : "+v"(sl));
      const uint32_t vo = (uint32_t)((sl >> 3) & 7) * tok + 16u * (uint32_t)(sl & 7);
      const __amdgpu_buffer_rsrc_t r8k = block_rsrc(t, kbase), r8v = block_rsrc(t, vbase);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma16(r8k, k8 + (16 * wave + 8 * i) * kRow8, vo + 8u * i * tok, 0);
        dma16(r8v, v8 + (16 * wave + 8 * i) * kRow8, vo + 8u * i * tok, 0);
      }
    };
    // convert: bf16 chunk c = tid + 256 j of each tile (row c / 16, chunk
    // c % 16) from the staged row's bytes 8 (c % 16) .. + 7, stored at the
    // swizzled chunk position the halves read
    auto convert8 = [&]() {
      int sl = threadIdx.x;
      asm volatile("" : "+v"(sl));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = sl + 256 * j;
        const int r = c >> 4, ch = c & 15;
        const u32x2 kb8 = *(const u32x2*)(k8 + r * kRow8 + 8 * ch);
        const u32x2 vb8 = *(const u32x2*)(v8 + r * kRow8 + 8 * ch);
        *(u32x4*)(kt0 + r * kRowBytes + 16 * (ch ^ kswz(r))) = fp8x8_to_bf16(kb8[0], kb8[1]);
        *(u32x4*)(vt0 + r * kRowBytes + 16 * (ch ^ vswz(r))) = fp8x8_to_f16(vb8[0], vb8[1]);
      }
    };
    stage8(0);
    for (int t = 0; t < ntiles; ++t) {
      wait_vmem<0>();
      __syncthreads();                     // tile t staged in Y; X free
      convert8();
      __syncthreads();                     // X holds tile t; Y free
      if (t + 1 < ntiles) stage8(t + 1);
      if (t < t_act) {
        const int k1 = kv_begin + t * kPrefillKeys + 32;
        const bool h1 = k1 < kv_end && (!causal || k1 <= pos_hi);
        const bool masked = t >= t_mask;
        half(t, 0, kt0, vt0, masked, nothing, nothing);
        if (h1) half(t, 1, kt0, vt0, masked, nothing, nothing);
      }
    }
  } else {
    for (int t = 0; t < ntiles; t += 2) {
      body(t, std::integral_constant<int, 0>{});
      if (t + 1 < ntiles) body(t + 1, std::integral_constant<int, 1>{});
    }
  }

  // epilogue: lanes l and l^32 hold the same query row of a block
  auto finish = [&](const f32x16 (&o)[4], float m, float l, bool ok, int r) {
    const float l_tot = sum_x32(l);
    if (!ok) return;
    const float inv = l_tot > 0.0f ? vsc / l_tot : 0.0f;
    const float lse2 = l_tot > 0.0f ? m + log2_(l_tot) : kNegInf;
    if (part < 0) {
      uint16_t* const o_dst = dec_item ? a.o_decode : a.o_prefill;
      float* const lse_dst = dec_item ? a.lse_decode : a.lse_prefill;
      uint16_t* op = o_dst + ((int64_t)(qrow0 + r) * a.hq + head) * kHeadDim + 4 * hl;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x2 w = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                           pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
          *(u32x2*)(op + 32 * db + 8 * g4) = w;
        }
      if (hl == 0 && lse_dst) lse_dst[(int64_t)(qrow0 + r) * a.hq + head] = lse2 * kLn2;
    } else {
      // fp32 partial (already divided by its own l): the merge reweights
      // partials whose sizes may differ by orders of magnitude, so they keep
      // full precision until the final rounding
      const int pi = part + hidx * (kPrefillRows / a.p_heads) + r;
      float* pp = a.part_o + (int64_t)pi * kHeadDim + 4 * hl;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(f32x4*)(pp + 32 * db + 8 * g4) =
              f32x4{o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv,
                    o[db][4 * g4 + 3] * inv};
      if (hl == 0) a.part_lse[pi] = lse2;
    }
  };
  // a restaged last tile may still be landing: LDS is reused after the item
  wait_vmem<0>();
  finish(oa, ma, la, okA, rA);
  finish(ob, mb, lb, okB, rB);
}

// ---------------------------------------------------------------------------
// Decode: one wavefront, <=16 query heads sharing a KV head, keys [kb, ke),
// 32 keys per step.  K goes straight from HBM into MFMA operand registers; V
// goes by LDS DMA into the wave's double-buffered slice and is read back
// transposed.  The loads of step s+1 are in flight while step s computes.
// With `ahead` set, lane 0 takes a ticket of that queue counter in the
// unit's second-to-last step, right after the last V DMA (so the last step's
// wait for its V covers the ticket too) and returns it in `ticket`; the
// caller's next claim then costs no round trip of its own.
//
// PACKED (queries packed by shared prefix, [PAT] abstract): the tile's rows
// are the query heads of several decode requests -- row j is head
// h0 + j % rpr of request members[D_QROW + j / rpr] (rpr = min(g, 16)) -- and
// every row writes a partial, at D_PART + (j / rpr) Hq D_PSTRIDE + (j % rpr)
// D_PSTRIDE.
// ---------------------------------------------------------------------------
template <int KVM, bool PACKED = false>
__device__ __forceinline__ void decode_unit(const KernelArgs& a, cptr it, char* __restrict__ vb0,
                                            char* __restrict__ vb1, int* ahead, int& ticket) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q4 = lane >> 4;
  const int qi = it[D_QROW], h0 = it[D_HEAD0], nq = it[D_NQ];
  const int kb = it[D_KV_BEGIN], ke = it[D_KV_END], kvreq = it[D_KVREQ];
  const int part = it[D_PART], pstride = it[D_PSTRIDE];
  const int kvh = h0 / a.group;
  const uint32_t tok = (uint32_t)a.hkv * kRowBytes;
  const char* kbase = (const char*)a.k + kvh * kRowBytes;
  const char* vbase = (const char*)a.v + kvh * kRowBytes;
  KvAddr<KVM> addr;
  addr.init(a, kvreq);
  const int span = ke - kb;
  const int nsteps = (span + kDecodeStep - 1) / kDecodeStep;
  const int nfull = span / kDecodeStep;

  // Q^T operand kk = 2h + p: lane holds query j (head h0 + j), d = 64h +
  // 16*q4 + 8p + e -- the d order of the K operands below
  u32x4 qf[4];
  {
    const bool ok = j < nq;
    const int jr = ok ? j : 0;
    const int qrow = PACKED ? ((cptr)a.d_members)[qi + jr / a.pack_rpr] : qi;
    const int qhead = PACKED ? h0 + jr % a.pack_rpr : h0 + jr;
    const uint16_t* qp = a.q_decode + ((int64_t)qrow * a.hq + qhead) * kHeadDim + 16 * q4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = ok ? *(const u32x4*)(qp + 64 * (kk >> 1) + 8 * (kk & 1)) : u32x4{0, 0, 0, 0};
  }

  // K: a 16-key block sb is fetched as four 1 KB loads, each of eight keys x
  // one whole 128-byte line (a load of 16 keys x 64 bytes would split every
  // line over two requests and halve the rate a CU can stream at).  Raw load
  // 4*sb + 2h + x: lane L reads key 8x + (L & 7), 16-byte chunk 8h + ((L >> 3)
  // ^ x).  kop() turns the pair x = 0, 1 into MFMA operands of 16 keys x 32 d.
  // V: LDS rows 4i + L/16 (i = 0..7) of the step's slice, chunk L%16.
  // A step's two 16-key blocks each lie in one page (page_size >= 16), so each
  // has one uniform buffer resource; in a unit's last step the blocks and the
  // lanes' rows are clamped to the last key (finite data, never read past it).
  const int dq = lane >> 4, dc = lane & 15;
  const int lastb = (ke - 1) & ~15;                 // start of the block holding key ke-1
  struct Blk { __amdgpu_buffer_rsrc_t rk, rv; int rmax; };
  auto block = [&](int s, int sb) {
    const int bs = min(kb + s * kDecodeStep + 16 * sb, lastb);
    const int64_t rw = addr.block_row(bs);
    return Blk{rsrc(kbase + rw * tok), rsrc(vbase + rw * tok), ke - 1 - bs};
  };
  const int k8 = lane & 7, kc = lane >> 3;
  auto load_k = [&](int s, u32x4 (&kr)[8]) {
    if (KVM != KV_PAGED_NARROW) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const Blk bl = block(s, sb);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t vk = (uint32_t)min(8 * x + k8, bl.rmax) * tok + 16u * (kc ^ x);
#pragma unroll
          for (int h = 0; h < 2; ++h) kr[4 * sb + 2 * h + x] = bload<kStream>(bl.rk, vk + 128u * h, 0);
        }
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int tk = min(kb + s * kDecodeStep + 16 * sb + 8 * x + k8, ke - 1);
          const char* pk = kbase + addr.row(tk) * tok + 16 * (kc ^ x);
#pragma unroll
          for (int h = 0; h < 2; ++h) kr[4 * sb + 2 * h + x] = gload(pk + 128 * h);
        }
    }
  };
  // MFMA operand p of the raw pair (A: x = 0, B: x = 1): lane L gets key
  // L & 15 and chunk 8h + 2(L >> 4) + p.  p = 0: A in place, lanes 8-15 of
  // each row from B in place; p = 1: lanes 0-7 take A from 8 lanes up, lanes
  // 8-15 take B from 8 lanes down (DPP row shifts, bank masks pick the half).
  auto kop = [](const u32x4& A, const u32x4& B, int p) {
    u32x4 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (p == 0) {
        r[c] = (uint32_t)__builtin_amdgcn_update_dpp((int)A[c], (int)B[c], 0xE4, 0xF, 0xC, false);
      } else {
        const int t = __builtin_amdgcn_update_dpp(0, (int)A[c], 0x108, 0xF, 0x3, false);
        r[c] = (uint32_t)__builtin_amdgcn_update_dpp(t, (int)B[c], 0x118, 0xF, 0xC, false);
      }
    }
    return r;
  };
  auto load_v = [&](int s, char* dst) {
    if (KVM != KV_PAGED_NARROW) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const Blk bl = block(s, sb);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = 4 * i4 + dq;
          const uint32_t vv = (uint32_t)min(r, bl.rmax) * tok + 16u * (dc ^ vswz(r));
          dma16<kStream>(bl.rv, dst + (16 * sb + 4 * i4) * kRowBytes, vv, 0);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + dq;
        const int tv = min(kb + s * kDecodeStep + r, ke - 1);
        *(u32x4*)(dst + 4 * i * kRowBytes + 16 * lane) =
            gload(vbase + addr.row(tv) * tok + 16 * (dc ^ vswz(r)));
      }
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf, l_run = 0.0f;
  const float sl2 = a.scale_log2;
  // V^T read lanes: rows 4*q4 + j/4 (+16), chunk 2 db + (j&3)/2, half j&1
  const int vrow0 = 4 * q4 + (j >> 2);
  const int vsw = vswz(vrow0);

  // Step s: S(s) from K(s) registers and softmax; V(s) read from LDS; then
  // the DMA of V(s+1) into the other buffer is issued and PV runs.  With
  // `more`, K(s+1) (8 loads) was requested after the DMA of V(s), so V(s) has
  // landed once at most 8 loads are outstanding.
  auto step = [&](int s, const u32x4 (&kr)[8], const char* vsrc, char* vnext, bool more) {
    // nothing is scheduled across a step's boundaries: the next step's
    // MFMAs hoisted into this one would wait for K loads still in flight
    __builtin_amdgcn_sched_barrier(0);
    const int k0 = kb + s * kDecodeStep;
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int h = kk >> 1, p = kk & 1;
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kop(kr[2 * h], kr[2 * h + 1], p)),
                                                   as_bf(qf[kk]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kop(kr[4 + 2 * h], kr[5 + 2 * h], p)),
                                                   as_bf(qf[kk]), s1, 0, 0, 0);
    }
    // s0[r]: key k0 + 4*q4 + r; s1[r]: key k0 + 16 + 4*q4 + r; query j
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r];
      x[4 + r] = s1[r];
    }
    if (s >= nfull) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + 4 * q4 + r >= ke) x[r] = kNegInf;
        if (k0 + 16 + 4 * q4 + r >= ke) x[4 + r] = kNegInf;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmax_(mx, x[r]);
    mx = max_x32(max_x16(mx));
    const float m_new = fmax_(m_run, mx * sl2);
    if (any_lane(m_new > m_run)) {
      const float alpha = exp2_(m_run - (m_new == kNegInf ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == kNegInf ? 0.0f : -m_run;
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x[r] = exp2_(__builtin_fmaf(x[r], sl2, nm));
      ls += x[r];
    }
    l_run += ls;
    // P^T operand: e = 0..3 -> key 4*q4 + e, e = 4..7 -> key 16 + 4*q4 + e - 4
    const u32x4 pb = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    const char* vt = vsrc + vrow0 * kRowBytes + 8 * (j & 1);
    if (more) wait_vmem<8>();
    else wait_vmem<0>();
    lds_fence();
    u32x4 af[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const char* cp = vt + 16 * ((2 * db + ((j & 3) >> 1)) ^ vsw);
      const u32x2 lo = tr_read(cp);
      const u32x2 hi = tr_read(cp + 16 * kRowBytes);
      af[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    lds_fence();
    if (more) load_v(s + 1, vnext);
    if (ahead != nullptr && s == nsteps - 2 && lane == 0) ticket = atomicAdd(ahead, 1);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(af[db]), as_bf(pb), o[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // The steady-state loop covers step pairs that both have a successor, so
  // every pass issues the same loads; the last one or two steps follow it.
  u32x4 ka[8], kn[8];
  if (nsteps > 0) {
    load_k(0, ka);
    load_v(0, vb0);
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
      load_k(s + 1, kn);
      step(s, ka, vb0, vb1, true);
      load_k(s + 2, ka);
      step(s + 1, kn, vb1, vb0, true);
    }
    if (s + 1 < nsteps) {
      load_k(s + 1, kn);
      step(s, ka, vb0, vb1, true);
      step(s + 1, kn, vb1, vb0, false);
    } else {
      step(s, ka, vb0, vb1, false);
    }
  }

  // epilogue: query j is spread over lanes j, j+16, j+32, j+48
  const float l_tot = sum_x32(sum_x16(l_run));
  if (j >= nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse2 = l_tot > 0.0f ? m_run + log2_(l_tot) : kNegInf;
  if (!PACKED && part < 0) {
    uint16_t* op = a.o_decode + ((int64_t)qi * a.hq + h0 + j) * kHeadDim + 4 * q4;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2 w = {pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                       pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
      *(u32x2*)(op + 16 * db) = w;
    }
    if (q4 == 0 && a.lse_decode) a.lse_decode[(int64_t)qi * a.hq + h0 + j] = lse2 * kLn2;
  } else {
    const int pi = PACKED ? part + (j / a.pack_rpr) * a.hq * pstride + (j % a.pack_rpr) * pstride
                          : part + j * pstride;
    float* pp = a.part_o + (int64_t)pi * kHeadDim + 4 * q4;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *(f32x4*)(pp + 16 * db) = f32x4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
                                      o[db][3] * inv};
    if (q4 == 0) a.part_lse[pi] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Shared-prefix tile ([PAT] abstract: queries packed by shared prefix so that
// the prefix's KV is loaded once, in a tile sized to the pack): a workgroup
// takes up to 64 rows -- row jr is query head h0 + jr % rpr of decode request
// members[D_QROW + jr / rpr], rpr = min(g, 16) -- over keys [kb, ke) of one
// KV head, read through request D_KVREQ's page table.  Wave w owns rows
// 16w .. 16w + 15 as one 16-row MFMA tile (the decode unit's step, with K
// read from LDS instead of registers); the four waves share every 32-key K/V
// step, which they stage together by LDS DMA (wave w: keys 8w .. 8w + 7 of
// the step) into double buffers, so each key's bytes leave HBM once per
// workgroup instead of once per 16 rows.  Every row writes a partial, at
// D_PART + (jr / rpr) Hq D_PSTRIDE + (jr % rpr) D_PSTRIDE.
//
// LDS: step buffers of parity 0 in X, of parity 1 in Y (K at +0, V at +8
// KiB).  K rows keep 16-byte chunk c at position c ^ (row & 15), so the
// sixteen keys of an MFMA operand read fall in sixteen distinct bank groups;
// V rows use the decode unit's layout.
// ---------------------------------------------------------------------------
template <int KVM>
__device__ __forceinline__ void prefix_tile(const KernelArgs& a, cptr it, char* __restrict__ bx,
                                            char* __restrict__ by) {
  const int lane = threadIdx.x & 63;
  const int wave = rfl(threadIdx.x >> 6);
  const int j = lane & 15, q4 = lane >> 4;
  const int qi = it[D_QROW], h0 = it[D_HEAD0], nq = it[D_NQ];
  const int kb = it[D_KV_BEGIN], ke = it[D_KV_END], kvreq = it[D_KVREQ];
  const int part = it[D_PART], pstride = it[D_PSTRIDE];
  const int rpr = a.pack_rpr;
  const int kvh = h0 / a.group;
  const uint32_t tok = (uint32_t)a.hkv * kRowBytes;
  const char* kbase = (const char*)a.k + kvh * kRowBytes;
  const char* vbase = (const char*)a.v + kvh * kRowBytes;
  KvAddr<KVM> addr;
  addr.init(a, kvreq);
  const int span = ke - kb;
  const int nsteps = (span + kDecodeStep - 1) / kDecodeStep;
  const int nfull = span / kDecodeStep;
  const int jr = 16 * wave + j;                      // tile row of this lane's query
  const bool active = 16 * wave < nq;                // wave-uniform

  // Q operand kk: lane holds query jr, d = 32 kk + 8 q4 .. + 7
  u32x4 qf[4];
  {
    const bool ok = jr < nq;
    const int jq = ok ? jr : 0;
    const int qrow = ((cptr)a.d_members)[qi + jq / rpr];
    const uint16_t* qp = a.q_decode + ((int64_t)qrow * a.hq + h0 + jq % rpr) * kHeadDim + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = ok ? *(const u32x4*)(qp + 32 * kk) : u32x4{0, 0, 0, 0};
  }

  // staging of step s: wave w deposits keys 8w + 4i + L/16 (i = 0, 1) of the
  // step, chunk position L%16, into the K and V halves of `buf`; the keys
  // lie in one 16-key block (page_size >= 16) whose rows are clamped to the
  // last key (finite data, never read past it)
  const int lastb = (ke - 1) & ~15;
  const int dq = lane >> 4, dc = lane & 15;
  auto stage = [&](int s, char* buf) {
    char* kd = buf + 8 * wave * kRowBytes;
    char* vd = buf + kDecStepBytes + 8 * wave * kRowBytes;
    if (KVM != KV_PAGED_NARROW) {
      const int bs = min(kb + s * kDecodeStep + 16 * (wave >> 1), lastb);
      const int64_t rw = addr.block_row(bs);
      const __amdgpu_buffer_rsrc_t rk = rsrc(kbase + rw * tok), rv = rsrc(vbase + rw * tok);
      const int rmax = ke - 1 - bs;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * (wave & 1) + 4 * i + dq;       // row in the 16-key block
        const int rs = 8 * wave + 4 * i + dq;             // row in the step
        const uint32_t ro = (uint32_t)min(r, rmax) * tok;
        dma16<kStream>(rk, kd + 4 * i * kRowBytes, ro + 16u * (dc ^ kswz(rs)), 0);
        dma16<kStream>(rv, vd + 4 * i * kRowBytes, ro + 16u * (dc ^ vswz(rs)), 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rs = 8 * wave + 4 * i + dq;
        const int64_t rw = addr.row(min(kb + s * kDecodeStep + rs, ke - 1));
        *(u32x4*)(kd + 4 * i * kRowBytes + 16 * lane) =
            gload(kbase + rw * tok + 16 * (dc ^ kswz(rs)));
        *(u32x4*)(vd + 4 * i * kRowBytes + 16 * lane) =
            gload(vbase + rw * tok + 16 * (dc ^ vswz(rs)));
      }
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf, l_run = 0.0f;
  const float sl2 = a.scale_log2;
  // K operand reads: key 16 sb + j, chunk 4 kk + q4 at position (4 kk + q4) ^ j
  // V^T read lanes: rows 4*q4 + j/4 (+16), chunk 2 db + (j&3)/2, half j&1
  const int vrow0 = 4 * q4 + (j >> 2);
  const int vsw = vswz(vrow0);

  auto step = [&](int s, const char* buf) {
    __builtin_amdgcn_sched_barrier(0);
    const int k0 = kb + s * kDecodeStep;
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const char* kp = buf + j * kRowBytes + 16 * ((4 * kk + q4) ^ j);
      const u32x4 ka = *(const u32x4*)kp;
      const u32x4 kc = *(const u32x4*)(kp + 16 * kRowBytes);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ka), as_bf(qf[kk]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kc), as_bf(qf[kk]), s1, 0, 0, 0);
    }
    // s0[r]: key k0 + 4*q4 + r; s1[r]: key k0 + 16 + 4*q4 + r; query jr
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r];
      x[4 + r] = s1[r];
    }
    if (s >= nfull) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + 4 * q4 + r >= ke) x[r] = kNegInf;
        if (k0 + 16 + 4 * q4 + r >= ke) x[4 + r] = kNegInf;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmax_(mx, x[r]);
    mx = max_x32(max_x16(mx));
    const float m_new = fmax_(m_run, mx * sl2);
    if (any_lane(m_new > m_run)) {
      const float alpha = exp2_(m_run - (m_new == kNegInf ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == kNegInf ? 0.0f : -m_run;
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x[r] = exp2_(__builtin_fmaf(x[r], sl2, nm));
      ls += x[r];
    }
    l_run += ls;
    const u32x4 pb = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    const char* vt = buf + kDecStepBytes + vrow0 * kRowBytes + 8 * (j & 1);
    u32x4 af[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const char* cp = vt + 16 * ((2 * db + ((j & 3) >> 1)) ^ vsw);
      const u32x2 lo = tr_read(cp);
      const u32x2 hi = tr_read(cp + 16 * kRowBytes);
      af[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(af[db]), as_bf(pb), o[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // step s reads the buffers of parity s & 1 (X or Y) while the DMAs of step
  // s + 1 fill the other object; the barrier at the top of a step makes the
  // whole step visible and frees the buffers the DMAs are about to refill
  stage(0, bx);
  for (int s = 0; s < nsteps; s += 2) {
    wait_vmem<0>();
    __syncthreads();
    if (s + 1 < nsteps) stage(s + 1, by);
    if (active) step(s, bx);
    if (s + 1 < nsteps) {
      wait_vmem<0>();
      __syncthreads();
      if (s + 2 < nsteps) stage(s + 2, bx);
      if (active) step(s + 1, by);
    }
  }
  // the buffers are reused by the workgroup's next unit
  __syncthreads();

  const float l_tot = sum_x32(sum_x16(l_run));
  if (jr >= nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse2 = l_tot > 0.0f ? m_run + log2_(l_tot) : kNegInf;
  const int pi = part + (jr / rpr) * a.hq * pstride + (jr % rpr) * pstride;
  float* pp = a.part_o + (int64_t)pi * kHeadDim + 4 * q4;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *(f32x4*)(pp + 16 * db) = f32x4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
                                    o[db][3] * inv};
  if (q4 == 0) a.part_lse[pi] = lse2;
}

// ---------------------------------------------------------------------------
// Decode over an FP8 E4M3 KV cache with one scale per KV head for K and for
// V ("Prefill vs. Decode GPU Utilization Imbalance", section "Quantization
// and compression as a lever on both the bandwidth and capacity problem"):
// half the bytes per key, the same unit and step structure as decode_unit.
// A token's row of one head is one 128-byte line.
//   K: whole lines into registers -- a 16-key block is two raw loads (x = 0,
//      1; lane L: key 8x + (L & 7), 16-byte chunk (L >> 3) ^ x) -- rebuilt
//      by kop() into 16 keys x one chunk (chunk 2r + p for the 16-lane row r)
//      and converted exactly to bf16: each chunk feeds two 16x16x32 MFMAs
//      over d = 16 (2r + p) + 8 half + e (Q is loaded in that order).  The K
//      scale multiplies the fp32 score together with sm_scale.
//   V: the same whole-line loads into registers, converted to bf16 and
//      written to the wave's LDS slice in decode_unit's layout (row = key,
//      swizzled 16-byte chunks), then read transposed as there; the V scale
//      multiplies the final O.
// A step's raw K and V of the next step are in flight while it computes.
// ---------------------------------------------------------------------------

template <int KVM>
__device__ __forceinline__ void decode_unit_fp8(const KernelArgs& a, cptr it, char* __restrict__ vbuf) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q4 = lane >> 4;
  const int qi = it[D_QROW], h0 = it[D_HEAD0], nq = it[D_NQ];
  const int kb = it[D_KV_BEGIN], ke = it[D_KV_END], kvreq = it[D_KVREQ];
  const int part = it[D_PART], pstride = it[D_PSTRIDE];
  const int kvh = h0 / a.group;
  constexpr uint32_t kRow8 = kHeadDim;               // bytes of one head's row
  const uint32_t tok = (uint32_t)a.hkv * kRow8;
  const char* kbase = (const char*)a.k + kvh * kRow8;
  const char* vbase = (const char*)a.v + kvh * kRow8;
  KvAddr<KVM> addr;
  addr.init(a, kvreq);
  const int span = ke - kb;
  const int nsteps = (span + kDecodeStep - 1) / kDecodeStep;
  const int nfull = span / kDecodeStep;
  // the scales (uniform per unit) through the scalar cache
  const float sl2 = a.scale_log2 * __builtin_bit_cast(float, ((cptr)a.k_scale)[kvh]);
  const float vsc = __builtin_bit_cast(float, ((cptr)a.v_scale)[kvh]);

  // Q operand kk = 2p + half: lane (query j, row q4) holds d = 32 q4 + 16 p + 8 half + e
  u32x4 qf[4];
  {
    const bool ok = j < nq;
    const uint16_t* qp = a.q_decode + ((int64_t)qi * a.hq + h0 + (ok ? j : 0)) * kHeadDim + 32 * q4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = ok ? *(const u32x4*)(qp + 8 * kk) : u32x4{0, 0, 0, 0};
  }

  const int lastb = (ke - 1) & ~15;
  const int k8 = lane & 7, kc = lane >> 3;
  struct Blk { __amdgpu_buffer_rsrc_t rk, rv; int rmax; };
  auto block = [&](int s, int sb) {
    const int bs = min(kb + s * kDecodeStep + 16 * sb, lastb);
    const int64_t rw = addr.block_row(bs);
    return Blk{rsrc(kbase + rw * tok), rsrc(vbase + rw * tok), ke - 1 - bs};
  };
  // raw loads of step s: k[2 sb + x] (chunk (L >> 3) ^ x), v[2 sb + x] (chunk L >> 3)
  auto load = [&](int s, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const Blk bl = block(s, sb);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t row = (uint32_t)min(8 * x + k8, bl.rmax) * tok;
        kr[2 * sb + x] = bload<kStream>(bl.rk, row + 16u * (kc ^ x), 0);
        vr[2 * sb + x] = bload<kStream>(bl.rv, row + 16u * kc, 0);
      }
    }
  };
  auto kop = [](const u32x4& A, const u32x4& B, int p) {
    u32x4 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (p == 0) {
        r[c] = (uint32_t)__builtin_amdgcn_update_dpp((int)A[c], (int)B[c], 0xE4, 0xF, 0xC, false);
      } else {
        const int t = __builtin_amdgcn_update_dpp(0, (int)A[c], 0x108, 0xF, 0x3, false);
        r[c] = (uint32_t)__builtin_amdgcn_update_dpp(t, (int)B[c], 0x118, 0xF, 0xC, false);
      }
    }
    return r;
  };

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf, l_run = 0.0f;
  const int vrow0 = 4 * q4 + (j >> 2);
  const int vsw = vswz(vrow0);

  auto step = [&](int s, const u32x4 (&kr)[4], const u32x4 (&vr)[4], bool more) {
    __builtin_amdgcn_sched_barrier(0);
    if (more) wait_vmem<8>();
    else wait_vmem<0>();
    // V(s): bf16 into the LDS slice (the previous step's transposed reads of
    // it were issued earlier; one wave's LDS operations stay in order)
    lds_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * (i >> 1) + 8 * (i & 1) + k8;          // key row of the step
      const u32x4 lo = fp8x8_to_bf16(vr[i][0], vr[i][1]);
      const u32x4 hi = fp8x8_to_bf16(vr[i][2], vr[i][3]);
      *(u32x4*)(vbuf + r * kRowBytes + 16 * ((2 * kc) ^ vswz(r))) = lo;
      *(u32x4*)(vbuf + r * kRowBytes + 16 * ((2 * kc + 1) ^ vswz(r))) = hi;
    }
    lds_fence();
    const int k0 = kb + s * kDecodeStep;
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const u32x4 c0 = kop(kr[0], kr[1], p);
      const u32x4 c1 = kop(kr[2], kr[3], p);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(fp8x8_to_bf16(c0[2 * hf], c0[2 * hf + 1])),
                                                     as_bf(qf[2 * p + hf]), s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(fp8x8_to_bf16(c1[2 * hf], c1[2 * hf + 1])),
                                                     as_bf(qf[2 * p + hf]), s1, 0, 0, 0);
      }
    }
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r];
      x[4 + r] = s1[r];
    }
    if (s >= nfull) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + 4 * q4 + r >= ke) x[r] = kNegInf;
        if (k0 + 16 + 4 * q4 + r >= ke) x[4 + r] = kNegInf;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmax_(mx, x[r]);
    mx = max_x32(max_x16(mx));
    const float m_new = fmax_(m_run, mx * sl2);
    if (any_lane(m_new > m_run)) {
      const float alpha = exp2_(m_run - (m_new == kNegInf ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == kNegInf ? 0.0f : -m_run;
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x[r] = exp2_(__builtin_fmaf(x[r], sl2, nm));
      ls += x[r];
    }
    l_run += ls;
    const u32x4 pb = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    const char* vt = vbuf + vrow0 * kRowBytes + 8 * (j & 1);
    u32x4 af[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const char* cp = vt + 16 * ((2 * db + ((j & 3) >> 1)) ^ vsw);
      const u32x2 lo = tr_read(cp);
      const u32x2 hi = tr_read(cp + 16 * kRowBytes);
      af[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    lds_fence();
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(af[db]), as_bf(pb), o[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  u32x4 ka[4], va[4], kn[4], vn[4];
  if (nsteps > 0) {
    load(0, ka, va);
    int s = 0;
    for (; s + 2 < nsteps; s += 2) {
      load(s + 1, kn, vn);
      step(s, ka, va, true);
      load(s + 2, ka, va);
      step(s + 1, kn, vn, true);
    }
    if (s + 1 < nsteps) {
      load(s + 1, kn, vn);
      step(s, ka, va, true);
      step(s + 1, kn, vn, false);
    } else {
      step(s, ka, va, false);
    }
  }

  // epilogue: query j is spread over lanes j, j+16, j+32, j+48; O carries
  // the V scale
  const float l_tot = sum_x32(sum_x16(l_run));
  if (j >= nq) return;
  const float inv = l_tot > 0.0f ? vsc / l_tot : 0.0f;
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
    for (int db = 0; db < 8; ++db)
      *(f32x4*)(pp + 16 * db) = f32x4{o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
                                      o[db][3] * inv};
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

__device__ __forceinline__ int* hot(const KernelArgs& a, int i) {
  return a.counters + i * kCtrStride;
}
__device__ __forceinline__ int peek(int* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Claims (one thread, for its workgroup).  A claim issues, all at once, the
// atomic on the caller's own pool or queue, reads of the other pools' or
// queues' counters, and a read of the other role's "empty" flag, so that it
// costs one round trip (microseconds under decode traffic) whether or not
// the caller's own queue still has work.  Only when the own queue is empty
// is an atomic spent on another one that still had work.  A caller that sees
// every queue of its role empty sets that role's flag and learns from
// *other_empty whether the other role was empty too (then it can exit).
//
// Prefill: one item per claim from the per-XCD pools (pool xcc first).
__device__ __forceinline__ int claim_prefill(const KernelArgs& a, int xcc, int* other_empty) {
  const int np = a.num_pools;
  const int p0 = xcc % np;
  const int k0 = atomicAdd(hot(a, CS_POOL + p0), 1);
  int seen[kMaxPools];
#pragma unroll
  for (int i = 1; i < kMaxPools; ++i)
    seen[i] = i < np ? peek(hot(a, CS_POOL + (xcc + i) % np)) : 0;
  const int oe = peek(hot(a, CS_EMPTY + 1));
  if (k0 < a.pool_off[p0 + 1] - a.pool_off[p0]) return a.pool_off[p0] + k0;
  for (int i = 1; i < kMaxPools; ++i) {
    if (i >= np) break;
    const int p = (xcc + i) % np;
    const int n = a.pool_off[p + 1] - a.pool_off[p];
    if (seen[i] >= n) continue;
    const int k = atomicAdd(hot(a, CS_POOL + p), 1);
    if (k < n) return a.pool_off[p] + k;
  }
  __hip_atomic_store(hot(a, CS_EMPTY + 0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *other_empty = oe;
  return -1;
}

// Decode: a group of kWavesPerWG consecutive units of the longest-first list,
// one per wave.  Groups are dealt round-robin to n_dq queues (queue q: groups
// q, q + n_dq, ..), so every queue is balanced and longest first too; q0 is
// one of the caller's XCD.  A workgroup's four waves start their units
// together, as in a grid launch of one group per workgroup, which measured
// faster than units taken one wave at a time (those keep every wave
// streaming to the very end).
//
// The own queue is empty: claim from the others (seen[i]: the counter of
// queue q0 + i as read earlier), else mark the role empty.
__device__ __forceinline__ int claim_decode_others(const KernelArgs& a, int q0, const int* seen,
                                                   int oe, int* other_empty) {
  const int nq = a.n_dq, ng = a.n_groups;
  for (int i = 1; i < kMaxDecodeQueues; ++i) {
    if (i >= nq) break;
    const int q = (q0 + i) % nq;
    if (q + nq * seen[i] >= ng) continue;
    const int g = q + nq * atomicAdd(hot(a, CS_DQ + q), 1);
    if (g < ng) return g;
  }
  __hip_atomic_store(hot(a, CS_EMPTY + 1), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *other_empty = oe;
  return -1;
}

__device__ __forceinline__ int claim_decode_group(const KernelArgs& a, int q0, int* other_empty) {
  const int nq = a.n_dq, ng = a.n_groups;
  const int g0 = q0 + nq * atomicAdd(hot(a, CS_DQ + q0), 1);
  int seen[kMaxDecodeQueues];
#pragma unroll
  for (int i = 1; i < kMaxDecodeQueues; ++i)
    seen[i] = i < nq ? peek(hot(a, CS_DQ + (q0 + i) % nq)) : ng;
  const int oe = peek(hot(a, CS_EMPTY + 0));
  if (g0 < ng) return g0;
  return claim_decode_others(a, q0, seen, oe, other_empty);
}

// The same claim with the own queue's ticket already taken (decode_unit's
// `ahead`): no round trip while that queue has work.
__device__ __forceinline__ int claim_decode_after(const KernelArgs& a, int q0, int ticket,
                                                  int* other_empty) {
  const int nq = a.n_dq, ng = a.n_groups;
  const int g0 = q0 + nq * ticket;
  if (g0 < ng) return g0;
  int seen[kMaxDecodeQueues];
#pragma unroll
  for (int i = 1; i < kMaxDecodeQueues; ++i)
    seen[i] = i < nq ? peek(hot(a, CS_DQ + (q0 + i) % nq)) : ng;
  const int oe = peek(hot(a, CS_EMPTY + 0));
  return claim_decode_others(a, q0, seen, oe, other_empty);
}

// First workgroup of a launch: zero the counter block of the next launch of
// this kind (not in use now; the previous user finished before this launch).
__device__ __forceinline__ void zero_next_counters(const KernelArgs& a) {
  if (a.counters_next == nullptr || blockIdx.x != 0) return;
  for (int i = threadIdx.x; i < kCtrSlots; i += blockDim.x) a.counters_next[i * kCtrStride] = 0;
  for (int i = threadIdx.x; i < kCuCounters; i += blockDim.x)
    a.counters_next[kCuCounterOff + i * kCellStride] = 0;
}

// Self-resetting launches (recorded into a graph): the last workgroup resets
// the counters, so that every replay starts from zero.  Completion is counted
// in two levels (8 groups by blockIdx, then the groups) to keep the
// per-address atomic traffic low.  Every claim a workgroup made returned
// before it counts itself done (each returned value was used), and each
// level's atomic is issued after the previous one returned, so no memory
// fence is needed.
__device__ __forceinline__ void finish_launch(const KernelArgs& a, int* s_last) {
  if (!a.self_reset) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = (int)blockIdx.x & 7;
    const int n_g = ((int)gridDim.x - g + 7) >> 3;
    int last = 0;
    if (atomicAdd(hot(a, CS_DONE + g), 1) == n_g - 1) {
      const int groups = min(8, (int)gridDim.x);
      last = atomicAdd(hot(a, CS_DONE_ALL), 1) == groups - 1;
    }
    *s_last = last;
  }
  __syncthreads();
  if (*s_last) {
    for (int i = threadIdx.x; i < kCtrSlots; i += blockDim.x)
      __hip_atomic_store(hot(a, i), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < kCuCounters; i += blockDim.x)
      __hip_atomic_store(&a.counters[kCuCounterOff + i * kCellStride], 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void trace_unit(const KernelArgs& a, int rec, int role, int unit,
                                           int slot, uint64_t t0) {
  pod_trace_record_t* r = a.trace + rec;
  r->block = (int)blockIdx.x;
  r->cu_slot = slot;
  r->role = role;
  r->unit = unit;
  r->t_start = t0;
  r->t_end = __builtin_amdgcn_s_memrealtime();
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
// The two LDS tile objects of a workgroup (see the LDS geometry note) and a
// few scheduling words.
#define POD_LDS_OBJECTS                                  \
  __shared__ __align__(16) char ldsx[2 * kTileBytes];    \
  __shared__ __align__(16) char ldsy[2 * kTileBytes];    \
  __shared__ int s_info[8];

// prefill tiles: K0, K1, V0, V1
#define POD_PREFILL_BUFFERS ldsx, ldsy, ldsx + kTileBytes, ldsy + kTileBytes
// decode wave w: step buffers of parity 0 / 1
#define POD_DECODE_BUFFERS(w)                                  \
  char* const db0 = ldsx + (w) * kDecStepBytes;               \
  char* const db1 = ldsy + (w) * kDecStepBytes;

// Fused kernel: one persistent launch of wgs_per_cu workgroups per CU.  A
// workgroup reads which CU it landed on, takes its first role from that CU's
// counter (prefill for its share of the CU's slots), and works through the
// queue of that role: prefill tiles one workgroup at a time, decode units in
// groups of four (one per wave).  When its queue runs dry it moves to the
// other queue, so no slot idles while work is left.  F8: an FP8 KV cache
// (the prefill tile's F8 form and the FP8 decode unit).
template <int KVM, bool ONE = false, bool F8 = false>
__global__ __launch_bounds__(256, 2) void pod_fused_kernel(KernelArgs a) {
  POD_LDS_OBJECTS
  const int tid = threadIdx.x;
  const int wave = rfl(tid >> 6), lane = tid & 63;
  zero_next_counters(a);
  if (tid == 0) {
    const int slot = cu_slot_id();
    int role;   // 0 prefill, 1 decode
    int* cell = &a.counters[kCuCounterOff + slot * kCellStride];
    const int tp = (a.prefill_quarters + (slot & 3)) >> 2;   // prefill target of this CU
    if (a.sched_mode == POD_SCHED_COLOCATE) {
      // the CU's workgroups start together: the ticket (arrival order on
      // this CU) gives the first tp of them the prefill role
      const int t = atomicAdd(cell, 1);
      role = (t % a.wgs_per_cu) < tp ? 0 : 1;
    } else if (a.sched_mode == POD_SCHED_SPLIT) {
      // the CU index within its shader array (0..7 or 0..15) spreads the
      // prefill CUs evenly over every array and die
      role = (slot & 7) < a.prefill_quarters ? 0 : 1;
    } else {
      role = 0;
    }
    s_info[0] = role;
    s_info[1] = slot;
  }
  __syncthreads();
  const int role0 = s_info[0], slot = s_info[1];
  const int xcc = slot >> 8;
  // ---- prefill tiles until the pools are empty.  A unit is claimed only
  // when the claimant is free (greedy list scheduling: the next unit goes to
  // the first worker to finish, which a claim made ahead of time would not
  // honour); a claim costs well under 1% of a unit. ----
  // Each phase returns whether the other role's queues were all seen empty
  // when its own ran out (then the workgroup is done).
  auto prefill_phase = [&]() -> bool {
    if (a.n_p == 0) return false;
    while (true) {
      __syncthreads();   // the previous unit / phase is done with LDS and s_info
      if (tid == 0) {
        int oe = 0;
        s_info[2] = claim_prefill(a, xcc, &oe);
        s_info[3] = oe;
      }
      __syncthreads();
      const int u = rfl(s_info[2]);
      if (u < 0) return rfl(s_info[3]) != 0;
      const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
      prefill_tile<KVM, false, F8>(a, (cptr)a.p_items + u * P_FIELDS, POD_PREFILL_BUFFERS);
      if (a.trace && tid == 0) trace_unit(a, u, 0, u, slot, t0);
    }
  };
  // ---- decode unit groups until the queues are empty: one unit per wave.
  // Wave 0 claims the next group as soon as its own unit is done, with the
  // ticket it took a step before that unit's end (a claim made at the end
  // costs a memory round trip, microseconds under decode traffic, in which
  // the four waves would idle; held for about a step, the claimed group
  // upsets no balance).  The claim goes to the s_info pair the current group
  // did not read, so the other waves may still be reading theirs. ----
  auto decode_phase = [&]() -> bool {
    if (a.n_d == 0) return false;
    POD_DECODE_BUFFERS(wave)
    const int q0 = (4 * xcc + (slot & 3)) % a.n_dq;   // one of this XCD's queues
    __syncthreads();   // the previous phase is done with LDS and s_info
    if (tid == 0) {
      int oe = 0;
      s_info[2] = claim_decode_group(a, q0, &oe);
      s_info[3] = oe;
    }
    int pair = 2;   // s_info pair holding the current claim: 2 or 5
    while (true) {
      __syncthreads();   // the claim is visible
      const int g = rfl(s_info[pair]);
      if (g < 0) return rfl(s_info[pair + 1]) != 0;
      const int u = g * kWavesPerWG + wave;   // wave 0's unit always exists
      int ticket = -1;
      if (u < a.n_d) {
        const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
        if constexpr (F8)
          decode_unit_fp8<KVM>(a, (cptr)a.d_items + u * D_FIELDS, db0);
        else
          decode_unit<KVM>(a, (cptr)a.d_items + u * D_FIELDS, db0, db1,
                           wave == 0 ? hot(a, CS_DQ + q0) : nullptr, ticket);
        if (a.trace && lane == 0) trace_unit(a, a.n_p + u, 1, u, slot, t0);
      }
      pair = 7 - pair;
      if (tid == 0) {
        int oe = 0;
        s_info[pair] = ticket >= 0 ? claim_decode_after(a, q0, ticket, &oe)
                                   : claim_decode_group(a, q0, &oe);
        s_info[pair + 1] = oe;
      }
    }
  };
  if constexpr (ONE) {
    // one unit of the workgroup's role (or of the other one when its own is
    // exhausted), then exit
    __syncthreads();
    if (tid == 0) {
      int oe = 0, u = -1, g = -1;
      const int q0 = (4 * xcc + (slot & 3)) % a.n_dq;
      if (role0 == 0 && a.n_p > 0) u = claim_prefill(a, xcc, &oe);
      if (u < 0 && a.n_d > 0) g = claim_decode_group(a, q0, &oe);
      if (u < 0 && g < 0 && role0 != 0 && a.n_p > 0) u = claim_prefill(a, xcc, &oe);
      s_info[2] = u;
      s_info[3] = g;
    }
    __syncthreads();
    const int u = rfl(s_info[2]), g = rfl(s_info[3]);
    if (u >= 0) {
      const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
      prefill_tile<KVM, false, F8>(a, (cptr)a.p_items + u * P_FIELDS, POD_PREFILL_BUFFERS);
      if (a.trace && tid == 0) trace_unit(a, u, 0, u, slot, t0);
    } else if (g >= 0) {
      POD_DECODE_BUFFERS(wave)
      const int du = g * kWavesPerWG + wave;
      if (du < a.n_d) {
        const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
        if constexpr (F8) {
          decode_unit_fp8<KVM>(a, (cptr)a.d_items + du * D_FIELDS, db0);
        } else {
          int ticket;
          decode_unit<KVM>(a, (cptr)a.d_items + du * D_FIELDS, db0, db1, nullptr, ticket);
        }
        if (a.trace && lane == 0) trace_unit(a, a.n_p + du, 1, du, slot, t0);
      }
    }
    finish_launch(a, &s_info[4]);
  } else {
    if (role0 == 0) {
      if (!prefill_phase()) decode_phase();
    } else {
      if (!decode_phase()) prefill_phase();
    }
    finish_launch(a, &s_info[4]);
  }
}

template <int KVM, bool BP = false, bool F8 = false>
__global__ __launch_bounds__(256, 2) void pod_prefill_kernel(KernelArgs a) {
  POD_LDS_OBJECTS
  zero_next_counters(a);
  if (threadIdx.x == 0) {
    int oe;
    s_info[0] = claim_prefill(a, cu_slot_id() >> 8, &oe);
  }
  __syncthreads();
  const int unit = s_info[0];
  __syncthreads();
  if (unit >= 0) {
    const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    prefill_tile<KVM, BP, F8>(a, (cptr)a.p_items + rfl(unit) * P_FIELDS, POD_PREFILL_BUFFERS);
    if (a.trace && threadIdx.x == 0) trace_unit(a, unit, 0, unit, cu_slot_id(), t0);
  }
  finish_launch(a, &s_info[1]);
}

template <int KVM>
__global__ __launch_bounds__(256, 2) void pod_decode_kernel(KernelArgs a) {
  POD_LDS_OBJECTS
  (void)s_info;
  const int wave = rfl(threadIdx.x >> 6);
  const int d = blockIdx.x * kWavesPerWG + wave;
  POD_DECODE_BUFFERS(wave)
  if (d < a.n_d) {
    const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    int ticket;
    decode_unit<KVM>(a, (cptr)a.d_items + d * D_FIELDS, db0, db1, nullptr, ticket);
    if (a.trace && (threadIdx.x & 63) == 0) trace_unit(a, a.n_p + d, 1, d, cu_slot_id(), t0);
  }
}

// Shared-prefix (packed) decode kernel: workgroups below n_p take one
// prefix tile each (the plan's p_items, in decode-item fields), the rest one
// group of four suffix units, one per wavefront (PAT-style plans).
template <int KVM>
__global__ __launch_bounds__(256, 2) void pod_decode_pack_kernel(KernelArgs a) {
  POD_LDS_OBJECTS
  (void)s_info;
  const int wave = rfl(threadIdx.x >> 6);
  if ((int)blockIdx.x < a.n_p) {
    prefix_tile<KVM>(a, (cptr)a.p_items + blockIdx.x * D_FIELDS, ldsx, ldsy);
    return;
  }
  const int d = ((int)blockIdx.x - a.n_p) * kWavesPerWG + wave;
  POD_DECODE_BUFFERS(wave)
  if (d < a.n_d) {
    int ticket;
    decode_unit<KVM, true>(a, (cptr)a.d_items + d * D_FIELDS, db0, db1, nullptr, ticket);
  }
}

// FP8-cache decode kernel: one group of four units per workgroup, one unit
// per wavefront (decode-only batches; every run path uses it).
template <int KVM>
__global__ __launch_bounds__(256, 2) void pod_decode_fp8_kernel(KernelArgs a) {
  POD_LDS_OBJECTS
  (void)s_info;
  (void)ldsy;
  const int wave = rfl(threadIdx.x >> 6);
  const int d = blockIdx.x * kWavesPerWG + wave;
  if (d < a.n_d) {
    const uint64_t t0 = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    decode_unit_fp8<KVM>(a, (cptr)a.d_items + d * D_FIELDS, ldsx + wave * kDecStepBytes);
    if (a.trace && (threadIdx.x & 63) == 0) trace_unit(a, a.n_p + d, 1, d, cu_slot_id(), t0);
  }
}

// Merge: one 16-lane group per (row, head) task, four tasks per wavefront.
// Every load of a task -- its split LSEs (lane j holds splits j, j + 16, ..)
// and its fp32 partial rows (16 lanes x 32 bytes = one 512-byte row) -- is
// issued before any arithmetic, so a task costs about one memory round trip.
// Splits are summed in index order.  With m_tasks == NULL the kernel merges
// a caller's dense [rows, merge_splits] partials (pod_attn_merge).
__global__ __launch_bounds__(256) void pod_merge_kernel(KernelArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int task = blockIdx.x * kMergeTasksPerWG + (threadIdx.x >> 6) * 4 + g;
  const bool live = task < a.n_m;
  int out, base, stride, n;
  bool is_dec;
  if (a.m_tasks != nullptr) {
    const u32x4 tf = *(const u32x4*)(a.m_tasks + (int64_t)(live ? task : 0) * M_FIELDS);
    out = (int)tf[M_OUT];
    base = (int)tf[M_BASE];
    stride = (int)tf[M_STRIDE];
    n = live ? (int)(tf[M_NFLAG] & 0xFFFFu) : 0;      // n <= 64
    is_dec = (tf[M_NFLAG] >> 16) != 0;
  } else {
    out = live ? task : 0;
    base = out * a.merge_splits;
    stride = 1;
    n = live ? a.merge_splits : 0;
    is_dec = false;
  }
  const float lsc = a.merge_lse_scale;
  float ls[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    ls[c] = 16 * c + j < n ? a.part_lse[base + (16 * c + j) * stride] * lsc : kNegInf;
  constexpr int kBatch = 8;
  const float* po = a.part_o + (int64_t)base * kHeadDim + 8 * j;
  f32x4 v0[kBatch], v1[kBatch];
  auto load_row = [&](int sp, int i) {
    if (sp < n) {
      const float* r = po + (int64_t)sp * stride * kHeadDim;
      v0[i] = *(const f32x4*)r;
      v1[i] = *(const f32x4*)(r + 4);
    } else {
      v0[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      v1[i] = v0[i];
    }
  };
#pragma unroll
  for (int i = 0; i < kBatch; ++i) load_row(i, i);
  // max and weight sum over the group's 16 lanes
  float m = fmax_(fmax_(ls[0], ls[1]), fmax_(ls[2], ls[3]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmax_(m, __shfl_xor(m, off));
  float wl[4], tot = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    wl[c] = (m == kNegInf || ls[c] == kNegInf) ? 0.0f : exp2_(ls[c] - m);   // 0: empty split
    tot += wl[c];
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  // the loop runs to the largest n of the wave's four tasks
  int nmax = n;
  nmax = max(nmax, __shfl_xor(nmax, 16));
  nmax = max(nmax, __shfl_xor(nmax, 32));
  nmax = rfl(nmax);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int s0 = 0; s0 < nmax; s0 += kBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) load_row(s0 + i, i);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int sp = s0 + i;                                   // uniform
      if (sp >= nmax) break;
      const float wsrc = sp < 16 ? wl[0] : sp < 32 ? wl[1] : sp < 48 ? wl[2] : wl[3];
      const float wgt = sp < n ? __shfl(wsrc, 16 * g + (sp & 15)) : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * v0[i][e];
        acc[4 + e] += wgt * v1[i][e];
      }
    }
  }
  if (!live) return;
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  uint16_t* o = (is_dec ? a.o_decode : a.o_prefill) + (int64_t)out * kHeadDim + 8 * j;
  *(u32x4*)o = u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  float* lse = is_dec ? a.lse_decode : a.lse_prefill;
  if (j == 0 && lse) lse[out] = tot > 0.0f ? (m + log2_(tot)) * kLn2 : kNegInf;
}

// HBM read-rate probe: workgroup b streams the contiguous chunk b of the
// buffer (so each walks its own pages in order), every lane with eight
// 16-byte non-temporal loads in flight, and folds the data into one word that
// is stored only if it matches `never` (no load is dead code, nothing is
// written).
__global__ __launch_bounds__(256) void pod_read_probe_kernel(const u32x4* __restrict__ p,
                                                             int64_t n16, uint32_t never,
                                                             uint32_t* sink) {
  const int64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = min(n16, lo + chunk);
  int64_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < hi; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == never) sink[0] = acc;
}

__global__ void pod_probe_kernel(int32_t* out) {
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = (int32_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
    out[2 * blockIdx.x + 1] = (int32_t)__builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20);
  }
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate device memory
// (pod_attn_plan_scratch): the plan's workspace -- counters, work lists and
// split partials -- lives in this array.  Each device holds its own copy for
// the life of the process.  In host code `scratch` names a host-side stand-in,
// never the device memory: the device address is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_address(int device, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
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

template <bool ONE, bool F8>
struct FusedK {
  template <int KVM>
  static void launch(int grid, hipStream_t s, const KernelArgs& a) {
    hipLaunchKernelGGL((pod_fused_kernel<KVM, ONE, F8>), dim3(grid), dim3(256), 0, s, a);
  }
};

// FP8 caches have pages of at least 16 tokens (or are contiguous), so the
// narrow-page form is not instantiated for them.
hipError_t launch_fused(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  auto go = [&](auto k) {
    using K = decltype(k);
    switch (kv_mode) {
      case KV_CONTIG: K::template launch<KV_CONTIG>(grid, s, a); break;
      case KV_PAGED_WIDE: K::template launch<KV_PAGED_WIDE>(grid, s, a); break;
      default: K::template launch<KV_PAGED_NARROW>(grid, s, a); break;
    }
  };
  auto go8 = [&](auto k) {
    using K = decltype(k);
    if (kv_mode == KV_CONTIG) K::template launch<KV_CONTIG>(grid, s, a);
    else K::template launch<KV_PAGED_WIDE>(grid, s, a);
  };
  if (a.kv_fp8) {
    if (kv_mode == KV_PAGED_NARROW) return hipErrorInvalidValue;
    if (a.one_unit) go8(FusedK<true, true>{});
    else go8(FusedK<false, true>{});
  } else if (a.one_unit) {
    go(FusedK<true, false>{});
  } else {
    go(FusedK<false, false>{});
  }
  return hipGetLastError();
}

template <bool BP, bool F8>
struct PrefillK {
  template <int KVM>
  static void launch(int grid, hipStream_t s, const KernelArgs& a) {
    hipLaunchKernelGGL((pod_prefill_kernel<KVM, BP, F8>), dim3(grid), dim3(256), 0, s, a);
  }
};

hipError_t launch_prefill(const KernelArgs& a, int kv_mode, int grid, hipStream_t s, bool batched) {
  auto go = [&](auto k) {
    using K = decltype(k);
    switch (kv_mode) {
      case KV_CONTIG: K::template launch<KV_CONTIG>(grid, s, a); break;
      case KV_PAGED_WIDE: K::template launch<KV_PAGED_WIDE>(grid, s, a); break;
      default: K::template launch<KV_PAGED_NARROW>(grid, s, a); break;
    }
  };
  if (a.kv_fp8) {
    // FP8: no narrow pages, no batched-prefill comparator (both refused by the planner)
    if (kv_mode == KV_PAGED_NARROW || batched) return hipErrorInvalidValue;
    if (kv_mode == KV_CONTIG) PrefillK<false, true>::launch<KV_CONTIG>(grid, s, a);
    else PrefillK<false, true>::launch<KV_PAGED_WIDE>(grid, s, a);
  } else if (batched) {
    go(PrefillK<true, false>{});
  } else {
    go(PrefillK<false, false>{});
  }
  return hipGetLastError();
}

hipError_t launch_decode(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  POD_DISPATCH(pod_decode_kernel, 0)
}

hipError_t launch_decode_pack(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  POD_DISPATCH(pod_decode_pack_kernel, 0)
}

hipError_t launch_decode_fp8(const KernelArgs& a, int kv_mode, int grid, hipStream_t s) {
  switch (kv_mode) {
    case KV_CONTIG:
      hipLaunchKernelGGL(pod_decode_fp8_kernel<KV_CONTIG>, dim3(grid), dim3(256), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL(pod_decode_fp8_kernel<KV_PAGED_WIDE>, dim3(grid), dim3(256), 0, s, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const KernelArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(pod_merge_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, int64_t n16, uint32_t never, uint32_t* sink,
                             int blocks, hipStream_t s) {
  hipLaunchKernelGGL(pod_read_probe_kernel, dim3(blocks), dim3(256), 0, s, (const u32x4*)buf, n16,
                     never, sink);
  return hipGetLastError();
}

hipError_t launch_probe(int32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(pod_probe_kernel, dim3(blocks), dim3(256), 0, s, out);
  return hipGetLastError();
}

}  // namespace pod
