// Kernel argument block shared by the run-side launcher (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace xattn {

struct AttnParams {
  const void* q;        // [total_q][hq][d]
  const void* k;        // [num_pages][page_size][hkv][d]
  const void* v;        // same layout as k
  void* out;            // [total_q][hq][d]
  float* lse;           // [total_q][hq] or nullptr
  float* ws_o;          // [ws_rows][d] fp32 partial outputs (normalised)
  float* ws_lse;        // [ws_rows] fp32 partial lse (natural log)
  const int32_t* reqs;  // [B][4]: qo_start, qo_len, kv_len, page_base
  const int32_t* units; // [n][8]: r, hk, row0, nrows, kv0, kv1, ws_row, cost
  const int32_t* pages; // [total_pages] physical page per logical page; nullptr: identity
  const int32_t* merges;// [m][4]: out_row, ws_row0, nchunks, stride
  // graph-stable launches: the grid is the slot's capacity and these device words hold
  // the plan's unit count of the launched family and its merge count (nullptr: the grid
  // size is the count)
  const int32_t* unit_count;
  const int32_t* merge_count;
  int32_t num_units;    // grid size of an attention launch
  int32_t num_merges;
  int32_t hq, hkv, d, group;
  int32_t page_size;
  int32_t page_shift;   // log2(page_size) when a power of two, else -1
  int32_t mask, block;
  int32_t tile_rows;    // query rows per MFMA tile unit (128 or 256)
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
  int64_t pool_bytes;   // bytes of each of the K and V pools (num_pages * page_size * hkv * d * elt)
};

// The tile kernel addresses K and V with 32-bit offsets from the pool base when the pools
// span less than 4 GB (every offset then fits).
inline bool buffer_loads_fit(const AttnParams& p) {
  return p.pool_bytes > 0 && p.pool_bytes <= static_cast<int64_t>(UINT32_MAX);
}

}  // namespace xattn
