// Host-side fuzz of the partitioner (test infrastructure): random batches, valid and
// invalid, through xattn::build_schedule, built with address and undefined-behaviour
// sanitizers. Every accepted schedule is checked against the invariants the kernels
// rely on. Prints "ok <cases> <accepted>" and exits 0, or names the first violation
// and exits 1.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <string>
#include <vector>

#include "partition.h"

namespace {

int violations = 0;

void check(bool ok, int it, const char* what) {
  if (!ok && violations++ == 0) std::fprintf(stderr, "case %d: %s\n", it, what);
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 2000;
  std::mt19937_64 rng(20261203);
  auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
  auto uni = [&](int lo, int hi) { return lo + static_cast<int>(rng() % static_cast<uint64_t>(hi - lo + 1)); };
  int accepted = 0;
  for (int it = 0; it < iters; ++it) {
    const int B = uni(0, 24);
    const int hkv = pick({1, 2, 4, 8});
    const int g = pick({1, 1, 2, 4, 8});
    const int hq = rng() % 50 == 0 ? hkv * g + 1 : hkv * g;
    const int dtype = uni(0, 1);
    const int d = rng() % 40 == 0 ? 48 : (dtype ? pick({64, 128}) : pick({16, 32, 64, 128}));
    const int ps = pick({1, 2, 3, 4, 16, 64});
    const int mask = uni(0, 2);
    const int block = uni(1, 130);
    std::vector<int32_t> qo(B), npg(B), last(B);
    for (int r = 0; r < B; ++r) {
      const int kv = rng() % 8 == 0 ? 0 : uni(1, rng() % 8 == 0 ? 9000 : 700);
      int q = rng() % 3 == 0 ? 1 : uni(0, 300);
      if (mask != 0 && q > kv) q = kv;
      qo[r] = q;
      npg[r] = kv == 0 ? 0 : (kv + ps - 1) / ps;
      last[r] = kv == 0 ? 1 : kv - (npg[r] - 1) * ps;
    }
    std::vector<int32_t> qo_indptr(B + 1, 0), kv_indptr(B + 1, 0);
    for (int r = 0; r < B; ++r) {
      qo_indptr[r + 1] = qo_indptr[r] + qo[r];
      kv_indptr[r + 1] = kv_indptr[r] + npg[r];
    }
    const int total_pages = kv_indptr[B];
    const int extra = uni(0, 5);
    std::vector<int32_t> pages(total_pages + extra);
    std::iota(pages.begin(), pages.end(), 0);
    std::shuffle(pages.begin(), pages.end(), rng);
    pages.resize(total_pages);
    const bool identity = rng() % 4 == 0;
    // a planted defect in some cases: the schedule must then be rejected, not crash
    const int defect = rng() % 10 == 0 ? uni(1, 4) : 0;
    const bool pass_last = rng() % 5 != 0;
    bool must_reject = false;
    if (defect == 1 && B > 1 && qo_indptr[1] != qo_indptr[B]) {
      std::swap(qo_indptr[1], qo_indptr[B]);
      must_reject = true;
    }
    if (defect == 2 && B > 0 && pass_last) {
      const int r = uni(0, B - 1);
      last[r] = ps + 1;
      must_reject = npg[r] > 0;
    }
    if (defect == 3 && total_pages > 0 && !identity) {
      pages[uni(0, total_pages - 1)] = total_pages + extra + 3;
      must_reject = true;
    }
    if (defect == 4 && B > 0) {
      kv_indptr[B] = kv_indptr[B - 1] - 1;
      must_reject = true;
    }

    xattn::PlanArgs a;
    a.qo_indptr = qo_indptr.data();
    a.kv_indptr = kv_indptr.data();
    a.kv_page_indices = identity ? nullptr : pages.data();
    a.kv_last_page_len = pass_last ? last.data() : nullptr;
    a.batch = B, a.hq = hq, a.hkv = hkv, a.d = d, a.page_size = ps;
    a.num_pages = total_pages + extra;
    a.mask = mask, a.block = block, a.sm_scale = 0.f, a.dtype = dtype;
    a.force_chunk = rng() % 3 == 0 ? uni(1, 400) : 0;
    a.tile_rows = pick({0, 0, 128, 256});
    xattn::Schedule s;
    std::string err;
    const int rc = xattn::build_schedule(a, s, err);
    if (rc != xattn::kOk) {
      check(!err.empty(), it, "rejected without a message");
      continue;
    }
    check(!must_reject, it, "a planted defect was accepted");
    ++accepted;
    check(s.reqs.size() == static_cast<size_t>(B) * 4, it, "reqs size");
    int64_t ws_units = 0;
    for (int f = 0; f < xattn::FAM_COUNT; ++f) {
      for (const xattn::Unit& u : s.units[f]) {
        check(u.r >= 0 && u.r < B, it, "unit request out of range");
        if (u.r < 0 || u.r >= B) continue;
        const int q = s.reqs[4 * u.r + 1], kv = s.reqs[4 * u.r + 2];
        check(u.hk >= 0 && u.hk < hkv, it, "unit kv head out of range");
        check(u.nrows >= 1 && u.row0 >= 0 && u.row0 + u.nrows <= q * (hq / hkv), it, "unit rows out of range");
        check(u.kv0 >= 0 && u.kv0 <= u.kv1 && u.kv1 <= kv, it, "unit keys out of range");
        const int rows_cap = f == xattn::FAM_F32 ? xattn::kF32Rows : f == xattn::FAM_DEC ? xattn::kDecMaxRows : s.tile_rows;
        check(u.nrows <= rows_cap, it, "unit holds more rows than its kernel");
        if (u.kv1 > u.kv0 && !s.identity) {
          const int npages = (u.kv1 - 1) / ps - u.kv0 / ps + 1;
          if (f == xattn::FAM_MMA) check(npages <= xattn::kMmaMaxPages, it, "tile unit spans too many pages");
          if (f == xattn::FAM_DEC) check(npages <= xattn::kDecMaxPages, it, "decode unit spans too many pages");
        }
        if (u.ws_row >= 0) {
          ++ws_units;
          check(static_cast<int64_t>(u.ws_row) + u.nrows <= s.ws_rows, it, "workspace row out of range");
        }
      }
    }
    for (const xattn::Merge& m : s.merges) {
      check(m.nchunks >= 2 && m.ws_row0 >= 0, it, "merge shape");
      check(static_cast<int64_t>(m.ws_row0) + static_cast<int64_t>(m.nchunks - 1) * m.stride < s.ws_rows, it,
            "merge reads past the workspace");
      check(m.out_row >= 0 && static_cast<int64_t>(m.out_row) < static_cast<int64_t>(qo_indptr[B]) * hq, it,
            "merge writes past the output");
    }
    check(s.merges.empty() == (ws_units == 0), it, "split units without merges, or merges without splits");
  }
  if (violations) {
    std::fprintf(stderr, "%d violations\n", violations);
    return 1;
  }
  std::printf("ok %d %d\n", iters, accepted);
  return 0;
}
