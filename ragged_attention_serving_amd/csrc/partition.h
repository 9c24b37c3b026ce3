// Host-side schedule for plan/run attention: validation, work partition, merge map.
// Pure C++17, no HIP: the same code builds the schedule that xattn_plan stages and
// the one xattn_schedule returns for inspection.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace xattn {

enum Family { FAM_F32 = 0, FAM_DEC = 1, FAM_MMA = 2, FAM_COUNT = 3 };

// Rows (query tokens x grouped heads) per unit for each family.
constexpr int kF32Rows = 4;    // fp32 kernel: scores of a chunk kept in LDS per row
// decode kernel: rows held in registers per lane. Units of 5-8 rows (8 query heads per KV
// head, or 2 tokens of 4) run faster as query tiles: the decode kernel's VALU work per key
// grows with its rows while its bytes do not.
constexpr int kDecMaxRows = 4;
constexpr int kMmaRows = 128;  // MFMA kernel, default: 4 waves x 32 query columns
constexpr int kF32MaxChunk = 1024;
// MFMA kernel: page indices of one unit staged in LDS; a unit may span at most this many pages
constexpr int kMmaMaxPages = 1024;
// decode kernel: page indices of one unit staged in LDS; a unit may span at most this many
constexpr int kDecMaxPages = 2048;
// XCDs of an MI355X: workgroup i of a launch is dispatched to XCD i % kXcds
constexpr int kXcds = 8;

struct PlanArgs {
  const int32_t* qo_indptr = nullptr;
  const int32_t* kv_indptr = nullptr;
  const int32_t* kv_page_indices = nullptr;
  const int32_t* kv_last_page_len = nullptr;
  int32_t batch = 0, hq = 0, hkv = 0, d = 0, page_size = 0;
  int64_t num_pages = 0;
  int32_t mask = 0, block = 0;
  float sm_scale = 0.f;
  int32_t dtype = 0;
  int32_t force_chunk = 0;  // > 0: split every context into chunks of this many keys
  int32_t tile_rows = 0;    // MFMA tile height, 128 or 256 (0: kMmaRows)
};

// One unit of work: a request's kv head, a range of its query rows, a KV range.
struct Unit {
  int32_t r, hk, row0, nrows, kv0, kv1, ws_row, cost;
};

// One output row assembled from split chunks by the merge kernel.
struct Merge {
  int32_t out_row, ws_row0, nchunks, stride;
};

struct Schedule {
  std::vector<int32_t> reqs;  // [B][4]: qo_start, qo_len, kv_len, page_base
  std::vector<Unit> units[FAM_COUNT];
  std::vector<Merge> merges;
  std::vector<int32_t> pages;  // copy of kv_page_indices (empty: identity table)
  std::vector<int32_t> kv_start;  // [B+1] cumulative context lengths (packed context rows)
  int64_t ws_rows = 0;
  int32_t dec_rows = 0;
  int32_t tile_rows = kMmaRows;
  int32_t chunk[FAM_COUNT] = {0, 0, 0};
  int64_t total_kv = 0;
  int64_t visible_pairs = 0;
  int32_t total_q = 0;
  int32_t group = 1;
  float scale = 0.f;
  bool identity = true;
};

// Status codes match xattn_status.
constexpr int kOk = 0, kErrInvalid = -1, kErrUnsupported = -2, kErrHip = -3, kErrOom = -4,
              kErrBusy = -5;

// Validates the arguments and fills `s`. Returns a status code; on error `err` says why
// and `s` is unspecified.
int build_schedule(const PlanArgs& a, Schedule& s, std::string& err);

// Last visible key index (inclusive) of query token qi in a request, before the KV
// range clip: -1 when it sees none.
int64_t last_visible_key(int mask, int block, int64_t qo_len, int64_t kv_len, int64_t qi);

}  // namespace xattn
