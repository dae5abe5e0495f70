// Host planner (see plan.h).
#include "plan.h"

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdio>
#include <numeric>

namespace pod {

namespace {

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pod_status_t fail(std::string* err, pod_status_t st, const char* fmt, long long a = 0,
                  long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b);
  if (err) *err = buf;
  return st;
}

// MI355X datasheet peaks used only to estimate the prefill share, with the
// fractions of them the kernels reach (measured: prefill 0.4-1 PFLOP/s,
// decode 5-6.4 TB/s).
constexpr double kPeakFlops = 2.5e15;   // dense bf16 MFMA, FLOP/s
constexpr double kPeakBytes = 8.0e12;   // HBM3E, B/s
constexpr double kPrefillEff = 0.30;    // expected fraction of MFMA peak
constexpr double kDecodeEff = 0.72;     // expected fraction of HBM peak

}  // namespace

pod_status_t validate(const pod_attn_params_t* p, int32_t np, const int32_t* qo,
                      const int32_t* pkv, int32_t nd, const int32_t* dkv,
                      const pod_attn_tuning_t* t, std::string* err) {
  if (!p) return fail(err, POD_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_qo_heads < 1 || p->num_kv_heads < 1)
    return fail(err, POD_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (got %lld, %lld)",
                p->num_qo_heads, p->num_kv_heads);
  if (p->num_qo_heads % p->num_kv_heads != 0)
    return fail(err, POD_ERR_INVALID_ARGUMENT,
                "num_qo_heads (%lld) is not a multiple of num_kv_heads (%lld)",
                p->num_qo_heads, p->num_kv_heads);
  if (p->head_dim != kHeadDim)
    return fail(err, POD_ERR_UNSUPPORTED, "head_dim %lld unsupported (only 128)", p->head_dim);
  if (p->kv_layout != POD_KV_CONTIGUOUS && p->kv_layout != POD_KV_PAGED)
    return fail(err, POD_ERR_INVALID_ARGUMENT, "kv_layout %lld invalid", p->kv_layout);
  if (p->kv_layout == POD_KV_PAGED && (!is_pow2(p->page_size) || p->page_size > 1024))
    return fail(err, POD_ERR_INVALID_ARGUMENT,
                "page_size %lld must be a power of two in [1, 1024]", p->page_size);
  if (p->causal != 0 && p->causal != 1)
    return fail(err, POD_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %lld)", p->causal);
  if (!(std::isfinite(p->sm_scale) && p->sm_scale > 0.0f))
    return fail(err, POD_ERR_INVALID_ARGUMENT, "sm_scale must be finite and > 0");
  if (p->kv_dtype != POD_KV_BF16 && p->kv_dtype != POD_KV_FP8_E4M3)
    return fail(err, POD_ERR_INVALID_ARGUMENT, "kv_dtype %lld invalid", p->kv_dtype);
  if (p->kv_dtype == POD_KV_FP8_E4M3) {
    if (p->kv_layout == POD_KV_PAGED && p->page_size < 16)
      return fail(err, POD_ERR_UNSUPPORTED, "FP8 KV caches need pages of >= 16 tokens (%lld)",
                  p->page_size);
  }
  if (np < 0 || nd < 0)
    return fail(err, POD_ERR_INVALID_ARGUMENT, "negative request count (%lld, %lld)", np, nd);
  if (np > 0 && (!qo || !pkv))
    return fail(err, POD_ERR_INVALID_ARGUMENT, "prefill length arrays are NULL");
  if (nd > 0 && !dkv)
    return fail(err, POD_ERR_INVALID_ARGUMENT, "decode length array is NULL");
  const int64_t kMaxLen = int64_t(1) << 24;
  int64_t sum_qo = 0;
  for (int32_t i = 0; i < np; ++i) {
    if (qo[i] < 1) return fail(err, POD_ERR_INVALID_ARGUMENT,
                               "prefill %lld: qo_len %lld < 1", i, qo[i]);
    if (pkv[i] < qo[i]) return fail(err, POD_ERR_INVALID_ARGUMENT,
                                    "prefill %lld: kv_len < qo_len (kv %lld)", i, pkv[i]);
    if (pkv[i] > kMaxLen) return fail(err, POD_ERR_UNSUPPORTED,
                                      "prefill %lld: kv_len %lld too large", i, pkv[i]);
    sum_qo += qo[i];
  }
  for (int32_t i = 0; i < nd; ++i) {
    if (dkv[i] < 1) return fail(err, POD_ERR_INVALID_ARGUMENT,
                                "decode %lld: kv_len %lld < 1", i, dkv[i]);
    if (dkv[i] > kMaxLen) return fail(err, POD_ERR_UNSUPPORTED,
                                      "decode %lld: kv_len %lld too large", i, dkv[i]);
  }
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (sum_qo * p->num_qo_heads > lim || int64_t(nd) * p->num_qo_heads > lim)
    return fail(err, POD_ERR_UNSUPPORTED, "too many (row, head) outputs");
  if (t) {
    if (t->wgs_per_cu != 0 && t->wgs_per_cu != 2)
      return fail(err, POD_ERR_UNSUPPORTED, "wgs_per_cu %lld unsupported (0 or 2)",
                  t->wgs_per_cu);
    if (t->prefill_quarters_per_cu < -1 || t->prefill_quarters_per_cu > 8)
      return fail(err, POD_ERR_INVALID_ARGUMENT, "prefill_quarters_per_cu %lld out of [-1, 8]",
                  t->prefill_quarters_per_cu);
    if (t->prefill_kv_splits < 0 || t->decode_kv_splits < 0)
      return fail(err, POD_ERR_INVALID_ARGUMENT, "negative forced split count");
    if (t->sched_mode < 0 || t->sched_mode > POD_SCHED_SPLIT)
      return fail(err, POD_ERR_INVALID_ARGUMENT, "sched_mode %lld invalid", t->sched_mode);
    if (t->match_sequential != 0 && t->match_sequential != 1)
      return fail(err, POD_ERR_INVALID_ARGUMENT, "match_sequential must be 0 or 1");
    if (p->kv_dtype == POD_KV_FP8_E4M3 && (t->flags & POD_FLAG_BATCHED_PREFILL))
      return fail(err, POD_ERR_UNSUPPORTED, "the batched-prefill comparator reads bf16 caches only");
  }
  return POD_OK;
}

namespace {
// Estimated prefill and decode times (s) at the expected fractions of the peaks.
void estimate_times(const Batch& b, double* tp, double* td) {
  const auto& p = b.params;
  double pairs_p = 0.0, keys_d = 0.0;
  for (size_t i = 0; i < b.qo.size(); ++i) {
    double q = b.qo[i], k = b.pkv[i];
    pairs_p += p.causal ? q * (k - q) + q * (q + 1) / 2 : q * k;
  }
  for (int32_t k : b.dkv) keys_d += k;
  const double f = 4.0 * kHeadDim * p.num_qo_heads * pairs_p;
  const double elem = p.kv_dtype == POD_KV_FP8_E4M3 ? 1.0 : 2.0;   // bytes per K or V element
  const double by = keys_d * p.num_kv_heads * kHeadDim * 2.0 * elem;
  *tp = f / (kPeakFlops * kPrefillEff);
  *td = by / (kPeakBytes * kDecodeEff);
}
}  // namespace

double prefill_share_estimate(const Batch& b) {
  double tp = 0.0, td = 0.0;
  estimate_times(b, &tp, &td);
  return tp + td > 0.0 ? tp / (tp + td) : 0.0;
}

int32_t auto_prefill_quarters(const Batch& b, int32_t wgs_per_cu, int32_t sched_mode) {
  const int32_t full = 4 * wgs_per_cu;
  if (b.qo.empty()) return 0;
  if (b.dkv.empty()) return full;
  double tp = 0.0, td = 0.0;
  estimate_times(b, &tp, &td);
  // rounded down: a prefill CU too many starves the decode, whose rate per CU
  // is capped, while one too few only delays the prefill until the decode
  // CUs join it (FP8 70B layer: 5 against 6 eighths, 1,431 against 1,667 us;
  // FP8 llama3-8b: 4 against 5, 136 against 147 us; every bf16 layer's choice
  // is the same either way)
  int32_t q = (int32_t)std::floor(full * tp / (tp + td));
  // SPLIT: between 3 and 6 eighths of the CUs start on prefill.  Fewer
  // prefill CUs make the prefill run long beside a decode that cannot use the
  // extra CUs (a CU's decode rate is capped by its own load issue, and HBM by
  // the sum): on the llama2-7b layer 3 beat 2 by 2-7%.  With several prefill
  // requests at least 4 eighths start on prefill (unless the estimate puts
  // the prefill under 1/16 of the time).  This is fitted to measurements, not
  // derived: on the batched mix (four prefill requests) 4 beat 3 by 1-7% at
  // 32-192 decodes and tied at 256, while on the one-request layers the
  // estimate's own choice held (llama3-8b: 3 stayed 1-2% ahead of 4).
  // COLOCATE: at least one prefill and one decode quarter.
  if (sched_mode == POD_SCHED_SPLIT) {
    const bool several = b.qo.size() > 1;
    const int32_t lo = several && 16.0 * tp >= tp + td ? 4 : 3;
    return std::min(full - 2, std::max(lo, q));
  }
  return std::min(full - 1, std::max(1, q));
}

void build_lists(const Batch& b, const pod_device_desc_t& dev, int64_t prefill_slots,
                 int32_t p_half_items_per_slot, int64_t decode_wave_slots, int32_t d_units_per_slot,
                 int32_t force_p_splits, int32_t force_d_splits, WorkLists* out,
                 bool decodes_as_prefill) {
  const auto& p = b.params;
  const int32_t hq = p.num_qo_heads, hkv = p.num_kv_heads, g = hq / hkv;
  const int32_t np = (int32_t)b.qo.size(), nd = (int32_t)b.dkv.size();
  WorkLists w;
  int64_t n_partials = 0;   // checked against the int32 indices at the end

  // ---- prefill items (request, group of nh query heads, block of npos
  // positions); nh * npos = kPrefillRows ----
  const int32_t nh = prefill_heads(g), npos = prefill_positions(g);
  struct Tile { int32_t qrow0, head, nrows, pos0, kv_end, req, kvh; };
  std::vector<Tile> tiles;
  int32_t qrow = 0;
  for (int32_t r = 0; r < np; ++r) {
    const int32_t qo = b.qo[r], kv = b.pkv[r];
    for (int32_t h = 0; h < hq; h += nh)
      for (int32_t r0 = 0; r0 < qo; r0 += npos) {
        Tile t;
        t.qrow0 = qrow + r0;
        t.head = h;
        t.nrows = std::min(npos, qo - r0);
        t.pos0 = kv - qo + r0;
        t.kv_end = p.causal ? std::min(kv, t.pos0 + t.nrows) : kv;
        t.req = r;
        t.kvh = h / g;
        tiles.push_back(t);
      }
    qrow += qo;
  }
  if (decodes_as_prefill) {
    for (int32_t i = 0; i < nd; ++i)
      for (int32_t h = 0; h < hq; h += nh) {
        const int32_t kv = b.dkv[i];
        tiles.push_back(Tile{i, h, 1, kv - 1, kv, np + i, h / g});
      }
  }
  // order: KV head major, so that one XCD pool holds the tiles sharing K/V
  std::stable_sort(tiles.begin(), tiles.end(), [](const Tile& a, const Tile& c) {
    return a.kvh < c.kvh;
  });
  int32_t s_all = 1;
  if (force_p_splits > 0) {
    s_all = std::min(force_p_splits, kMaxMergeSplits);
  } else if (!tiles.empty()) {
    // [POD] "Cap prefill splitting": a few waves of items over the slots at
    // most (the caller's count per slot; one for a sequential launch).
    s_all = (int32_t)std::max<int64_t>(
        1, (std::max(1, p_half_items_per_slot) * prefill_slots) / (2 * (int64_t)tiles.size()));
    s_all = std::min(s_all, kMaxPrefillSplits);
  }
  struct PI { std::array<int32_t, P_FIELDS> f; double work; };
  std::vector<PI> pitems;
  {
    // room for every merge task (at most one per prefill row and head, one
    // per decode and head), so that filling the lists never reallocates
    int64_t rows = 0;
    for (int32_t x : b.qo) rows += x;
    w.m_tasks.reserve((size_t)M_FIELDS * (size_t)((rows + nd) * hq));
  }
  for (const Tile& t : tiles) {
    const int32_t n_kt = (int32_t)ceil_div(t.kv_end, kPrefillKeys);
    int32_t s = std::max(1, std::min(s_all, n_kt));
    const int32_t per = (int32_t)ceil_div(n_kt, s);
    s = (int32_t)ceil_div(n_kt, per);
    int32_t base = -1;
    const bool dec_tile = t.req >= np;
    if (s > 1) {
      base = (int32_t)n_partials;
      n_partials += s * kPrefillRows;
      const size_t at = w.m_tasks.size();
      w.m_tasks.resize(at + (size_t)M_FIELDS * nh * t.nrows);
      int32_t* q = w.m_tasks.data() + at;
      const int32_t flags = s | (dec_tile ? 1 << 16 : 0);
      for (int32_t j = 0; j < nh; ++j)
        for (int32_t i = 0; i < t.nrows; ++i, q += M_FIELDS) {
          q[0] = (t.qrow0 + i) * hq + t.head + j;
          q[1] = base + j * npos + i;
          q[2] = kPrefillRows;
          q[3] = flags;
        }
    }
    w.p_splits_max = std::max(w.p_splits_max, s);
    for (int32_t k = 0; k < s; ++k) {
      const int32_t kb = k * per * kPrefillKeys;
      const int32_t ke = std::min(t.kv_end, (k + 1) * per * kPrefillKeys);
      PI it;
      it.f = {t.qrow0, t.head, t.nrows, t.pos0, kb, ke, t.req,
              base < 0 ? -1 : base + k * kPrefillRows};
      static_assert(P_FIELDS == 8, "prefill item fields");
      // a wave computes its 64 rows whatever the valid count, so a one-row
      // decode tile costs a full wave per head (batched prefill only; the
      // tuned lists keep the valid-row estimate)
      const double rows = dec_tile || decodes_as_prefill
                              ? double(nh) * kWaveRows * ceil_div(t.nrows, kWaveRows)
                              : double(t.nrows);
      it.work = rows * double(ke - kb);
      pitems.push_back(std::move(it));
    }
  }
  // ---- XCD pools: contiguous runs of the KV-head-ordered list, equal work ----
  const int32_t nx = std::max(1, std::min(dev.num_xcds, kMaxXcds));
  double total = 0.0;
  for (auto& it : pitems) total += it.work;
  w.pool_off.assign(nx + 1, 0);
  {
    double acc = 0.0;
    int32_t x = 0;
    for (size_t i = 0; i < pitems.size(); ++i) {
      // item i goes to pool x where x = floor(acc_mid / share)
      const double mid = acc + 0.5 * pitems[i].work;
      int32_t want = total > 0 ? (int32_t)std::floor(mid * nx / total) : 0;
      want = std::min(nx - 1, std::max(x, want));
      while (x < want) w.pool_off[++x] = (int32_t)i;
      acc += pitems[i].work;
    }
    while (x < nx) w.pool_off[++x] = (int32_t)pitems.size();
  }
  // longest first within each pool (a pool shares its K/V whatever the
  // order): causal row blocks grow with position, and in tile order the
  // longest items would be claimed last and lengthen the tail
  for (int32_t x = 0; x < nx; ++x)
    std::stable_sort(pitems.begin() + w.pool_off[x], pitems.begin() + w.pool_off[x + 1],
                     [](const PI& a, const PI& c) { return a.work > c.work; });
  w.p_items.reserve(pitems.size() * P_FIELDS);
  for (auto& it : pitems) w.p_items.insert(w.p_items.end(), it.f.begin(), it.f.end());

  // ---- decode units (request, KV head, <=16 query heads, split) ----
  const int32_t qchunks = (int32_t)ceil_div(g, kDecodeRows);
  double total_keys = 0.0;
  for (int32_t k : b.dkv) total_keys += double(k) * hkv * qchunks;
  int64_t chunk =
      total_keys >= double(decode_wave_slots) * kMinDecodeChunk ? kMinDecodeChunk : kMinDecodeChunkSmall;
  if (decode_wave_slots > 0 && total_keys > 0) {
    const int64_t c =
        (int64_t)std::ceil(total_keys / double(std::max(1, d_units_per_slot) * decode_wave_slots));
    chunk = std::max<int64_t>(chunk, ceil_div(c, kDecodeStep) * kDecodeStep);
  }
  struct DI { std::array<int32_t, D_FIELDS> f; int32_t work; };
  std::vector<DI> ditems;
  for (int32_t i = 0; i < (decodes_as_prefill ? 0 : nd); ++i) {
    const int32_t kv = b.dkv[i];
    const int32_t steps = (int32_t)ceil_div(kv, kDecodeStep);
    int64_t s64 = force_d_splits > 0
                      ? std::min(force_d_splits, kMaxMergeSplits)
                      : std::min<int64_t>(ceil_div(kv, chunk), kMaxDecodeSplits);
    int32_t s = (int32_t)std::max<int64_t>(1, std::min<int64_t>(s64, steps));
    const int32_t per = (int32_t)ceil_div(steps, s);
    s = (int32_t)ceil_div(steps, per);
    int32_t region = -1;
    if (s > 1) {
      region = (int32_t)n_partials;
      n_partials += (int64_t)hq * s;
      for (int32_t h = 0; h < hq; ++h) {
        w.m_tasks.push_back(i * hq + h);
        w.m_tasks.push_back(region + h * s);
        w.m_tasks.push_back(1);
        w.m_tasks.push_back(s | (1 << 16));
      }
    }
    w.d_splits_max = std::max(w.d_splits_max, s);
    for (int32_t kh = 0; kh < hkv; ++kh)
      for (int32_t qc = 0; qc < qchunks; ++qc) {
        const int32_t h0 = kh * g + qc * kDecodeRows;
        const int32_t nq = std::min(kDecodeRows, g - qc * kDecodeRows);
        for (int32_t k = 0; k < s; ++k) {
          const int32_t kb = k * per * kDecodeStep;
          const int32_t ke = std::min(kv, (k + 1) * per * kDecodeStep);
          DI it;
          it.f = {i, h0, nq, kb, ke, np + i, region < 0 ? -1 : region + h0 * s + k,
                  region < 0 ? 0 : s};
          it.work = ke - kb;
          ditems.push_back(it);
        }
      }
  }
  // longest first: claimed in this order, the last units to start are the
  // shortest (and the four waves of a sequential decode workgroup get similar work)
  std::stable_sort(ditems.begin(), ditems.end(),
                   [](const DI& a, const DI& c) { return a.work > c.work; });
  w.d_items.reserve(ditems.size() * D_FIELDS);
  for (auto& it : ditems) w.d_items.insert(w.d_items.end(), it.f.begin(), it.f.end());
  // partial indices are int32 (work-list fields and kernel arithmetic): a
  // larger count marks the lists unusable (the caller refuses the plan)
  w.n_partials = n_partials <= INT32_MAX ? (int32_t)n_partials : -1;
  *out = std::move(w);
}

void build_prefix_lists(const Batch& b, const std::vector<int32_t>& group_of,
                        const std::vector<int32_t>& prefix_len, int64_t decode_wave_slots,
                        int32_t force_d_splits, WorkLists* out, std::vector<int32_t>* members) {
  const auto& p = b.params;
  const int32_t hq = p.num_qo_heads, hkv = p.num_kv_heads, g = hq / hkv;
  const int32_t nd = (int32_t)b.dkv.size();
  const int32_t rpr = std::min(g, kDecodeRows);         // tile rows of one member
  const int32_t qchunks = (int32_t)ceil_div(g, kDecodeRows);
  // members per prefix tile in a query-head chunk of nh heads: a partial
  // chunk (g > 16, not a multiple of 16) holds one member, so that row jr is
  // always head h0 + jr % rpr of member jr / rpr
  auto per_tile = [&](int32_t nh) { return nh == rpr ? kPrefixTileRows / rpr : 1; };
  // groups: the given ones (in order, members in decode order), then every
  // ungrouped decode as a group of one with no shared prefix
  struct G { std::vector<int32_t> m; int32_t plen; };
  std::vector<G> groups(prefix_len.size());
  for (size_t gi = 0; gi < prefix_len.size(); ++gi) groups[gi].plen = prefix_len[gi];
  for (int32_t i = 0; i < nd; ++i)
    if (group_of[i] >= 0) groups[group_of[i]].m.push_back(i);
  for (int32_t i = 0; i < nd; ++i)
    if (group_of[i] < 0) groups.push_back(G{{i}, 0});
  // Split lengths.  Suffix units: about two per decode wavefront, at least
  // kMinDecodeChunk keys (as decode units are sized).  Prefix tiles are
  // claimed first, so they take a share of the workgroup slots equal to
  // their share of the work, a tile's wave-key counted at kPrefixTileWeight
  // of a suffix unit's (its four waves share every K/V load): tile and
  // suffix work then end together.
  double tile_keys = 0.0, sfx_keys = 0.0;
  for (const G& gr : groups) {
    if (gr.m.empty()) continue;
    for (int32_t qc = 0; qc < qchunks; ++qc) {
      const int32_t nh = std::min(kDecodeRows, g - qc * kDecodeRows);
      tile_keys += double(gr.plen) * hkv * (double)ceil_div((int64_t)gr.m.size(), per_tile(nh));
    }
    for (int32_t r : gr.m) sfx_keys += double(b.dkv[r] - gr.plen) * hkv * qchunks;
  }
  const double tile_work = kPrefixTileWeight * kWavesPerWG * tile_keys;
  int64_t chunk = kMinDecodeChunk, chunk_p = kMinDecodeChunk;
  if (decode_wave_slots > 0 && tile_work + sfx_keys > 0) {
    const double keys = kWavesPerWG * tile_keys + sfx_keys;
    chunk = std::max<int64_t>(chunk, ceil_div((int64_t)std::ceil(keys / (2.0 * decode_wave_slots)),
                                              kDecodeStep) * kDecodeStep);
    const double wg_slots = double(decode_wave_slots) / kWavesPerWG;
    const double tiles = std::max(1.0, wg_slots * tile_work / (tile_work + sfx_keys));
    chunk_p = std::max<int64_t>(kDecodeStep, ceil_div((int64_t)std::ceil(tile_keys / tiles),
                                                      kDecodeStep) * kDecodeStep);
  }
  constexpr int32_t kMaxSegSplits = kMaxMergeSplits / 2;   // prefix + suffix <= 64
  auto splits_of = [&](int32_t len, int64_t ch) -> std::pair<int32_t, int32_t> {   // (count, keys per split)
    if (len <= 0) return {0, 0};
    const int32_t steps = (int32_t)ceil_div(len, kDecodeStep);
    int64_t s = force_d_splits > 0 ? force_d_splits : ceil_div(len, ch);
    s = std::max<int64_t>(1, std::min<int64_t>({s, (int64_t)kMaxSegSplits, (int64_t)steps}));
    const int32_t per = (int32_t)ceil_div(steps, s) * kDecodeStep;
    return {(int32_t)ceil_div(len, per), per};
  };
  WorkLists w;
  members->clear();
  int64_t n_partials = 0;   // checked against the int32 indices at the end
  struct DI { std::array<int32_t, D_FIELDS> f; int32_t work; };
  std::vector<DI> tiles, items;
  for (const G& gr : groups) {
    if (gr.m.empty()) continue;
    const int32_t moff = (int32_t)members->size();
    members->insert(members->end(), gr.m.begin(), gr.m.end());
    const auto [sp, pp] = splits_of(gr.plen, chunk_p);
    int32_t ss_max = 0;
    for (int32_t r : gr.m) ss_max = std::max(ss_max, splits_of(b.dkv[r] - gr.plen, chunk).first);
    const int32_t smax = sp + ss_max;
    const int32_t gbase = (int32_t)n_partials;
    n_partials += (int64_t)gr.m.size() * hq * smax;
    auto region = [&](int32_t rl, int32_t h) { return gbase + (rl * hq + h) * smax; };
    const int32_t nm = (int32_t)gr.m.size();
    for (int32_t kh = 0; kh < hkv; ++kh)
      for (int32_t qc = 0; qc < qchunks; ++qc) {
        const int32_t h0 = kh * g + qc * kDecodeRows;
        const int32_t nh = std::min(kDecodeRows, g - qc * kDecodeRows);
        const int32_t pt = per_tile(nh);
        // prefix: tiles of up to pt members
        for (int32_t m0 = 0; m0 < nm && gr.plen > 0; m0 += pt) {
          const int32_t cnt = std::min(pt, nm - m0);
          for (int32_t k = 0; k < sp; ++k) {
            const int32_t kb = k * pp, ke = std::min(gr.plen, (k + 1) * pp);
            DI it;
            it.f = {moff + m0, h0, (cnt - 1) * rpr + nh, kb, ke, (int32_t)b.qo.size() + gr.m[0],
                    region(m0, h0) + k, smax};
            it.work = ke - kb;
            tiles.push_back(it);
          }
        }
        // suffixes
        for (int32_t rl = 0; rl < nm; ++rl) {
          const int32_t r = gr.m[rl];
          const auto [ss, ps] = splits_of(b.dkv[r] - gr.plen, chunk);
          for (int32_t k = 0; k < ss; ++k) {
            const int32_t kb = gr.plen + k * ps, ke = std::min(b.dkv[r], gr.plen + (k + 1) * ps);
            DI it;
            it.f = {moff + rl, h0, nh, kb, ke, (int32_t)b.qo.size() + r,
                    region(rl, h0) + sp + k, smax};
            it.work = ke - kb;
            items.push_back(it);
          }
        }
      }
    for (int32_t rl = 0; rl < nm; ++rl) {
      const int32_t n = sp + splits_of(b.dkv[gr.m[rl]] - gr.plen, chunk).first;
      for (int32_t h = 0; h < hq; ++h) {
        w.m_tasks.push_back(gr.m[rl] * hq + h);
        w.m_tasks.push_back(region(rl, h));
        w.m_tasks.push_back(1);
        w.m_tasks.push_back(n | (1 << 16));
      }
    }
    w.d_splits_max = std::max(w.d_splits_max, smax);
  }
  auto longest_first = [](const DI& a, const DI& c) { return a.work > c.work; };
  std::stable_sort(tiles.begin(), tiles.end(), longest_first);
  std::stable_sort(items.begin(), items.end(), longest_first);
  for (auto& it : tiles) w.p_items.insert(w.p_items.end(), it.f.begin(), it.f.end());
  for (auto& it : items) w.d_items.insert(w.d_items.end(), it.f.begin(), it.f.end());
  w.pool_off = {0, w.n_p()};
  // partial indices are int32 (work-list fields and kernel arithmetic): a
  // larger count marks the lists unusable (the caller refuses the plan)
  w.n_partials = n_partials <= INT32_MAX ? (int32_t)n_partials : -1;
  *out = std::move(w);
}

}  // namespace pod
