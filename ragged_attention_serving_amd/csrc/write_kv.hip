// Context write: each request's keys and values, packed (length, heads, head_dim) in
// request order, go into the slots of its pages, once, before attention reads them.
//
// One block per (request, group of kTokens context positions). A block copies the rows
// of its positions in both pools: a position's row (all KV heads, Hkv * D elements) is
// contiguous in the packed source and in its page slot, so the copy runs over 16-byte
// chunks of rows; every thread has several chunks of K and V in flight. Blocks past a
// request's context length exit at once. Slots past kv_len in a last page, and pages
// of no request, are never written.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kTokens = 16;   // context positions per block
constexpr int kThreads = 256;
constexpr int kUnroll = 4;    // chunks per thread per round

__global__ __launch_bounds__(kThreads) void write_kv_kernel(WriteParams w) {
  const int r = blockIdx.x / w.groups;
  const int* rq = w.reqs + 4 * r;
  const int kv_len = rq[2], page_base = rq[3];
  const int t0 = (blockIdx.x - r * w.groups) * kTokens;
  if (t0 >= kv_len) return;
  const int nt = min(kTokens, kv_len - t0);
  const int cpr = w.row_bytes >> 4;  // 16-byte chunks per row
  const int total = nt * cpr;
  const int64_t src_row0 = static_cast<int64_t>(w.kv_start[r]) + t0;
  const char* ks = static_cast<const char*>(w.k_src);
  const char* vs = static_cast<const char*>(w.v_src);
  char* kd = static_cast<char*>(w.k_pages);
  char* vd = static_cast<char*>(w.v_pages);

  for (int base = 0; base < total; base += kThreads * kUnroll) {
    uint4 kx[kUnroll], vx[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = base + u * kThreads + threadIdx.x;
      dst[u] = -1;
      if (c < total) {
        const int tt = c / cpr, ch = c - tt * cpr;
        const int t = t0 + tt;
        const int lp = w.page_shift >= 0 ? (t >> w.page_shift) : (t / w.page_size);
        const int slot = t - lp * w.page_size;
        const int page = w.pages ? w.pages[page_base + lp] : page_base + lp;
        dst[u] = (static_cast<int64_t>(page) * w.page_size + slot) * w.row_bytes + 16 * ch;
        const int64_t src = (src_row0 + tt) * w.row_bytes + 16 * ch;
        kx[u] = *reinterpret_cast<const uint4*>(ks + src);
        vx[u] = *reinterpret_cast<const uint4*>(vs + src);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (dst[u] >= 0) {
        *reinterpret_cast<uint4*>(kd + dst[u]) = kx[u];
        *reinterpret_cast<uint4*>(vd + dst[u]) = vx[u];
      }
    }
  }
}

}  // namespace

int write_kv_groups(int max_kv_len) { return (max_kv_len + kTokens - 1) / kTokens; }

hipError_t launch_write_kv(const WriteParams& w, const Launch& l) {
  if (w.batch == 0 || w.groups <= 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(w.batch) * w.groups)), block(kThreads);
  void* args[] = {const_cast<WriteParams*>(&w)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(write_kv_kernel), grid, block, args, 0,
                            l.stream, l.start, l.stop, 0);
}

}  // namespace xattn
