// Launchers for the gfx950 kernels (each defined next to its kernel).
#pragma once

#include <hip/hip_runtime.h>

#include "params.h"

namespace xattn {

// Where a kernel goes: the stream and, when timing, two events that the runtime stamps
// with the kernel's own start and end (hipExtLaunchKernel), so that the measured time is
// the kernel's alone, with no launch gap.
struct Launch {
  hipStream_t stream = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename Kernel>
hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, const AttnParams& p, const Launch& l) {
  void* args[] = {const_cast<AttnParams*>(&p)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, l.stream,
                            l.start, l.stop, 0);
}

// fp32 storage and arithmetic, any mask, head_dim 16/32/64/128; units of <= 4 rows.
hipError_t launch_attn_f32(const AttnParams& p, const Launch& l);
// bf16 decode: units of up to `rows` query rows sharing one KV head (rows in 1, 2, 4).
hipError_t launch_attn_decode(const AttnParams& p, int rows, const Launch& l);
// bf16 MFMA tiles: units of up to 128 query rows sharing one KV head.
hipError_t launch_attn_mma(const AttnParams& p, const Launch& l);
// log-sum-exp merge of split rows into out (dtype 0 fp32, 1 bf16) and lse.
hipError_t launch_merge(const AttnParams& p, int dtype, const Launch& l);

// Context write: packed per-request rows [sum kv_len][row_bytes] into their page slots.
struct WriteParams {
  const void* k_src;
  const void* v_src;
  void* k_pages;
  void* v_pages;
  const int32_t* reqs;      // [B][4] of the plan (kv_len at 2, page_base at 3)
  const int32_t* kv_start;  // [B+1] first packed row of each request
  const int32_t* pages;     // page table, nullptr: identity
  int32_t batch;
  int32_t groups;           // blocks per request: write_kv_groups(max kv_len)
  int32_t page_size;
  int32_t page_shift;       // log2(page_size) when a power of two, else -1
  int32_t row_bytes;        // Hkv * head_dim * element size (a multiple of 16)
};
int write_kv_groups(int max_kv_len);
hipError_t launch_write_kv(const WriteParams& w, const Launch& l);

// The static device scratch of xattn_run_noalloc: its size in bytes, and the current
// device's address of it (resolved once per device, then cached).
size_t static_scratch_bytes();
hipError_t static_scratch(float** ptr);

}  // namespace xattn
