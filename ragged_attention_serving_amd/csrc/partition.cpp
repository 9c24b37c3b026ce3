// Host-side schedule: validation, partition into units, KV chunking and merge map.
//
// Inputs follow the query packing of page "mstar.engine.resources.attn.cross"
// (QueryPacking: requests in packed order plus cumulative query lengths) and a CSR
// page table over the context (FlashInferCrossManager reads the context as an
// ordinary paged KV stream). Long contexts are split into KV chunks spread across
// compute units; split rows are put back together by a log-sum-exp merge.
#include "partition.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <numeric>

namespace xattn {

int64_t last_visible_key(int mask, int block, int64_t qo_len, int64_t kv_len, int64_t qi) {
  if (kv_len <= 0) return -1;
  const int64_t pos = kv_len - qo_len + qi;  // this query's key position
  switch (mask) {
    case 0:
      return kv_len - 1;
    case 1:
      return std::min(pos, kv_len - 1);
    default: {
      const int64_t end = (pos / block + 1) * block;  // first key of the next block
      return std::min(end, kv_len) - 1;
    }
  }
}

static int fail(std::string& err, int code, const std::string& msg) {
  err = msg;
  return code;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }


// Workgroup i of a launch runs on XCD i % kXcds (round-robin dispatch). Groups of units
// that share a (request, KV head) are assigned whole to one XCD (greedy, largest group
// first, to the least loaded XCD that still has room), each group's units back to back
// in that XCD's sequence, largest first; position p of the launch then takes the next
// unit of XCD p % kXcds.
static void order_for_xcds(std::vector<Unit>& units) {
  const int64_t n = static_cast<int64_t>(units.size());
  if (n <= kXcds) {
    std::stable_sort(units.begin(), units.end(), [](const Unit& x, const Unit& y) { return x.cost > y.cost; });
    return;
  }
  std::stable_sort(units.begin(), units.end(), [](const Unit& x, const Unit& y) {
    if (x.r != y.r) return x.r < y.r;
    if (x.hk != y.hk) return x.hk < y.hk;
    return x.cost > y.cost;
  });
  struct Group {
    int64_t begin, end, cost;
  };
  std::vector<Group> groups;
  for (int64_t i = 0; i < n;) {
    int64_t j = i, c = 0;
    while (j < n && units[j].r == units[i].r && units[j].hk == units[i].hk) c += units[j++].cost;
    groups.push_back(Group{i, j, c});
    i = j;
  }
  std::stable_sort(groups.begin(), groups.end(), [](const Group& a, const Group& b) { return a.cost > b.cost; });
  int64_t cap[kXcds], load[kXcds];
  std::vector<Unit> queue[kXcds];
  for (int x = 0; x < kXcds; ++x) {
    cap[x] = (n - x + kXcds - 1) / kXcds;
    load[x] = 0;
  }
  for (const Group& gr : groups) {
    int64_t left = gr.end - gr.begin, at = gr.begin;
    while (left > 0) {
      int best = -1;
      for (int x = 0; x < kXcds; ++x)
        if (cap[x] >= left && (best < 0 || load[x] < load[best])) best = x;
      if (best < 0)  // no XCD has room for the rest of the group: use the emptiest
        for (int x = 0; x < kXcds; ++x)
          if (cap[x] > 0 && (best < 0 || cap[x] > cap[best])) best = x;
      const int64_t take = std::min(left, cap[best]);
      for (int64_t k = 0; k < take; ++k) {
        load[best] += units[at].cost;
        queue[best].push_back(units[at++]);
      }
      cap[best] -= take;
      left -= take;
    }
  }
  std::vector<Unit> out(n);
  for (int64_t p = 0; p < n; ++p) out[p] = queue[p % kXcds][p / kXcds];
  units.swap(out);
}

int build_schedule(const PlanArgs& a, Schedule& s, std::string& err) {
  s = Schedule();
  const int B = a.batch;
  if (B < 0) return fail(err, kErrInvalid, "batch_size < 0");
  if (B > 0 && (!a.qo_indptr || !a.kv_indptr))
    return fail(err, kErrInvalid, "qo_indptr and kv_indptr are required");
  if (a.hq < 1 || a.hkv < 1) return fail(err, kErrInvalid, "head counts must be >= 1");
  if (a.hq % a.hkv != 0) return fail(err, kErrInvalid, "num_qo_heads % num_kv_heads != 0");
  if (a.page_size < 1) return fail(err, kErrInvalid, "page_size < 1");
  if (a.mask < 0 || a.mask > 2) return fail(err, kErrInvalid, "unknown mask_mode");
  if (a.mask == 2 && a.block < 1) return fail(err, kErrInvalid, "block_size < 1 for BLOCK_CAUSAL");
  if (a.dtype != 0 && a.dtype != 1) return fail(err, kErrInvalid, "unknown dtype");
  if (a.dtype == 0 && a.d != 16 && a.d != 32 && a.d != 64 && a.d != 128)
    return fail(err, kErrUnsupported, "fp32 head_dim must be 16, 32, 64 or 128");
  if (a.dtype == 1 && a.d != 64 && a.d != 128)
    return fail(err, kErrUnsupported, "bf16 head_dim must be 64 or 128");
  if (a.force_chunk < 0) return fail(err, kErrInvalid, "force_chunk < 0");
  if (a.tile_rows != 0 && a.tile_rows != 128 && a.tile_rows != 256)
    return fail(err, kErrInvalid, "tile_rows must be 128 or 256");
  s.tile_rows = a.tile_rows ? a.tile_rows : kMmaRows;
  // the kernels take the scale in log2 units: it must stay finite there
  if (std::isnan(a.sm_scale) || (a.sm_scale > 0.f && !std::isfinite(a.sm_scale * 1.4426950408889634f)))
    return fail(err, kErrInvalid, "sm_scale must be finite (<= 0 selects 1/sqrt(head_dim))");

  const int g = a.hq / a.hkv;
  s.group = g;
  s.scale = a.sm_scale > 0.f ? a.sm_scale : 1.0f / std::sqrt(static_cast<float>(a.d));
  s.identity = a.kv_page_indices == nullptr;

  // ---- validate the packing and the page table, collect per-request lengths
  if (B > 0 && (a.qo_indptr[0] != 0 || a.kv_indptr[0] != 0))
    return fail(err, kErrInvalid, "qo_indptr[0] and kv_indptr[0] must be 0");
  s.reqs.resize(static_cast<size_t>(B) * 4);
  s.kv_start.assign(static_cast<size_t>(B) + 1, 0);
  for (int r = 0; r < B; ++r) {
    const int64_t qo = static_cast<int64_t>(a.qo_indptr[r + 1]) - a.qo_indptr[r];
    const int64_t np = static_cast<int64_t>(a.kv_indptr[r + 1]) - a.kv_indptr[r];
    if (qo < 0) return fail(err, kErrInvalid, "qo_indptr decreases at request " + std::to_string(r));
    if (np < 0) return fail(err, kErrInvalid, "kv_indptr decreases at request " + std::to_string(r));
    int64_t kv = 0;
    if (np > 0) {
      int64_t last = a.page_size;
      if (a.kv_last_page_len) {
        last = a.kv_last_page_len[r];
        if (last < 1 || last > a.page_size)
          return fail(err, kErrInvalid,
                      "kv_last_page_len out of [1, page_size] at request " + std::to_string(r));
      }
      kv = (np - 1) * a.page_size + last;
      if (kv > INT32_MAX) return fail(err, kErrInvalid, "context longer than 2^31-1 keys");
    }
    if (a.mask != 0 && qo > kv)
      return fail(err, kErrInvalid,
                  "causal masks need qo_len <= kv_len (request " + std::to_string(r) + ")");
    s.reqs[4 * r + 0] = a.qo_indptr[r];
    s.reqs[4 * r + 1] = static_cast<int32_t>(qo);
    s.reqs[4 * r + 2] = static_cast<int32_t>(kv);
    s.reqs[4 * r + 3] = a.kv_indptr[r];
    s.total_kv += kv;
    // (context rows past 2^31 are not addressable by the context write; plan still works)
    s.kv_start[r + 1] = static_cast<int32_t>(std::min<int64_t>(s.total_kv, INT32_MAX));
  }
  s.total_q = B > 0 ? a.qo_indptr[B] : 0;
  if (static_cast<int64_t>(s.total_q) * a.hq > INT32_MAX)
    return fail(err, kErrInvalid, "too many query rows");
  const int64_t total_pages = B > 0 ? a.kv_indptr[B] : 0;
  if (total_pages > 0 && a.num_pages < 1) return fail(err, kErrInvalid, "num_pages is required");
  if (s.identity) {
    if (total_pages > a.num_pages && total_pages > 0)
      return fail(err, kErrInvalid, "identity page table runs past num_pages");
  } else if (total_pages > 0) {
    s.pages.assign(a.kv_page_indices, a.kv_page_indices + total_pages);
    for (int64_t i = 0; i < total_pages; ++i) {
      const int32_t p = s.pages[i];
      if (p < 0 || p >= a.num_pages)
        return fail(err, kErrInvalid, "kv_page_indices[" + std::to_string(i) + "] out of range");
    }
  }

  // ---- classify requests and size the work per family
  // Requests with few query rows (tokens x grouped heads) go to the decode kernel, the
  // rest to the MFMA tile kernel. In a batch whose KV traffic is mostly prefill, the few
  // short requests ride along in the tile launch instead (one launch, no second kernel).
  bool small_to_tiles = false;
  if (a.dtype != 0) {
    int64_t short_kv = 0, tile_kv = 0;
    for (int r = 0; r < B; ++r) {
      const int64_t qo = s.reqs[4 * r + 1], kv = s.reqs[4 * r + 2];
      if (qo == 0) continue;
      const int64_t rows = qo * g;
      if (rows <= kDecMaxRows) short_kv += kv;
      else tile_kv += kv * ((rows + s.tile_rows - 1) / s.tile_rows);
    }
    small_to_tiles = tile_kv > 0 && short_kv <= tile_kv;
  }
  auto family_of = [&](int64_t rows) -> int {
    if (a.dtype == 0) return FAM_F32;
    return rows <= kDecMaxRows && !small_to_tiles ? FAM_DEC : FAM_MMA;
  };
  auto rows_per_unit = [&](int fam) -> int64_t {
    return fam == FAM_F32 ? kF32Rows : fam == FAM_DEC ? kDecMaxRows : s.tile_rows;
  };
  // KV range [0, hi) a row tile needs: up to the last key its last row sees.
  auto tile_hi = [&](int r, int64_t row_end) -> int64_t {
    const int64_t qo = s.reqs[4 * r + 1], kv = s.reqs[4 * r + 2];
    const int64_t qi_max = (row_end - 1) / g;
    return last_visible_key(a.mask, a.block, qo, kv, qi_max) + 1;
  };

  int64_t fam_work[FAM_COUNT] = {0, 0, 0};   // key-heads (decode) or tile count (mma)
  int64_t fam_maxkv[FAM_COUNT] = {0, 0, 0};
  int64_t fam_units[FAM_COUNT] = {0, 0, 0};  // units before any split
  int dec_rows = 0;
  for (int r = 0; r < B; ++r) {
    const int64_t qo = s.reqs[4 * r + 1];
    if (qo == 0) continue;
    const int64_t rows = qo * g;
    const int fam = family_of(rows);
    const int64_t rpu = rows_per_unit(fam);
    if (fam == FAM_DEC) dec_rows = std::max<int>(dec_rows, static_cast<int>(rows));
    for (int64_t row0 = 0; row0 < rows; row0 += rpu) {
      const int64_t row_end = std::min(rows, row0 + rpu);
      const int64_t hi = tile_hi(r, row_end);
      fam_work[fam] += (fam == FAM_MMA ? 1 : hi) * a.hkv;
      fam_maxkv[fam] = std::max(fam_maxkv[fam], hi);
      fam_units[fam] += a.hkv;
    }
    // visible pairs: exact count per query row, for the metric
    const int64_t kv = s.reqs[4 * r + 2];
    for (int64_t qi = 0; qi < qo; ++qi)
      s.visible_pairs += (last_visible_key(a.mask, a.block, qo, kv, qi) + 1) * a.hq;
  }
  if (dec_rows > 0) {
    int R = 1;
    while (R < dec_rows) R *= 2;
    s.dec_rows = R;
  }

  // chunk length per family
  int64_t chunk[FAM_COUNT] = {0, 0, 0};
  for (int fam = 0; fam < FAM_COUNT; ++fam) {
    if (fam_maxkv[fam] == 0 && fam_work[fam] == 0) continue;
    int64_t c;
    if (a.force_chunk > 0) {
      c = a.force_chunk;
    } else if (fam == FAM_F32) {
      c = kF32MaxChunk;
    } else if (fam == FAM_DEC) {
      // The decode kernel keeps up to 8 workgroups resident per compute unit (2048 on the
      // chip). If the unsplit units fill the chip in one round and are about the same
      // length, they all start at once and finish together: no split, no merge.
      // Otherwise aim for about 2048 units (longer units run more efficiently, so the
      // chunk is not made any shorter than that needs).
      const int64_t mean = ceil_div(std::max<int64_t>(fam_work[fam], 1), std::max<int64_t>(fam_units[fam], 1));
      if (fam_units[fam] >= 1024 && fam_units[fam] <= 2048 && fam_maxkv[fam] * 4 <= mean * 5) {
        c = std::max<int64_t>(fam_maxkv[fam], 1);
      } else {
        c = std::max<int64_t>(256, round_up(ceil_div(std::max<int64_t>(fam_work[fam], 1), 2048), 64));
      }
    } else {
      // split only when there are too few query tiles to fill 256 compute units twice
      const int64_t tiles = std::max<int64_t>(fam_work[fam], 1);
      if (tiles >= 512) {
        c = std::max<int64_t>(fam_maxkv[fam], 1);
      } else {
        const int64_t f = ceil_div(512, tiles);
        c = std::max<int64_t>(256, round_up(ceil_div(fam_maxkv[fam], f), 64));
      }
    }
    if (fam == FAM_F32) c = std::min<int64_t>(c, kF32MaxChunk);
    // a paged MFMA unit stages its page indices in LDS: keep its span within kMmaMaxPages
    if (fam == FAM_MMA && !s.identity) c = std::min<int64_t>(c, static_cast<int64_t>(kMmaMaxPages - 2) * a.page_size);
    if (fam == FAM_DEC && !s.identity) c = std::min<int64_t>(c, static_cast<int64_t>(kDecMaxPages - 2) * a.page_size);
    c = std::min<int64_t>(std::max<int64_t>(c, 1), INT32_MAX);
    chunk[fam] = c;
    s.chunk[fam] = static_cast<int32_t>(c);
  }

  // ---- emit units and the merge map
  for (int r = 0; r < B; ++r) {
    const int64_t qo = s.reqs[4 * r + 1];
    if (qo == 0) continue;
    const int64_t qo_start = s.reqs[4 * r + 0];
    const int64_t rows = qo * g;
    const int fam = family_of(rows);
    const int64_t rpu = rows_per_unit(fam);
    for (int hk = 0; hk < a.hkv; ++hk) {
      for (int64_t row0 = 0; row0 < rows; row0 += rpu) {
        const int64_t row_end = std::min(rows, row0 + rpu);
        const int64_t nrows = row_end - row0;
        const int64_t hi = tile_hi(r, row_end);
        const int64_t nch = hi <= 0 ? 1 : ceil_div(hi, chunk[fam]);
        // equal chunks, rounded to whole 64-key tiles when that keeps the count; a forced
        // chunk length is taken as given
        int64_t step = hi <= 0 ? 1 : ceil_div(hi, nch);
        if (a.force_chunk > 0) step = chunk[fam];  // the forced length, after the caps above
        else if (nch > 1 && round_up(step, 64) <= chunk[fam] && ceil_div(hi, round_up(step, 64)) == nch)
          step = round_up(step, 64);
        int32_t base = -1;
        if (nch > 1) {
          if (s.ws_rows + nch * nrows > INT32_MAX) return fail(err, kErrInvalid, "workspace too large");
          base = static_cast<int32_t>(s.ws_rows);
          s.ws_rows += nch * nrows;
          for (int64_t rr = 0; rr < nrows; ++rr) {
            const int64_t row = row0 + rr;
            const int64_t tok = qo_start + row / g;
            const int64_t head = static_cast<int64_t>(hk) * g + row % g;
            s.merges.push_back(Merge{static_cast<int32_t>(tok * a.hq + head),
                                     static_cast<int32_t>(base + rr), static_cast<int32_t>(nch),
                                     static_cast<int32_t>(nrows)});
          }
        }
        for (int64_t c = 0; c < nch; ++c) {
          const int64_t k0 = hi <= 0 ? 0 : std::min(hi, c * step);
          const int64_t k1 = hi <= 0 ? 0 : std::min(hi, (c + 1) * step);
          Unit u;
          u.r = r;
          u.hk = hk;
          u.row0 = static_cast<int32_t>(row0);
          u.nrows = static_cast<int32_t>(nrows);
          u.kv0 = static_cast<int32_t>(k0);
          u.kv1 = static_cast<int32_t>(k1);
          u.ws_row = nch > 1 ? static_cast<int32_t>(base + c * nrows) : -1;
          const int64_t cost = (k1 - k0 + 64) * (fam == FAM_MMA ? (nrows + 31) / 32 : 1);
          u.cost = static_cast<int32_t>(std::min<int64_t>(cost, INT32_MAX));
          s.units[fam].push_back(u);
        }
      }
    }
  }

  // Decode units read disjoint KV: longest-processing-time first (the dispatcher hands
  // out workgroups in order, so the expensive units start early and the short ones fill
  // the tail). Tile units of one (request, KV head) re-read the same keys: keep each such
  // group on one XCD, back to back, so the re-reads hit that XCD's L2.
  std::stable_sort(s.units[FAM_DEC].begin(), s.units[FAM_DEC].end(),
                   [](const Unit& x, const Unit& y) { return x.cost > y.cost; });
  order_for_xcds(s.units[FAM_MMA]);
  order_for_xcds(s.units[FAM_F32]);
  return kOk;
}

}  // namespace xattn
