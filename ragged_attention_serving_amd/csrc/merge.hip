// Split-KV merge: rebuild an output row from the partial results of its KV chunks.
//
// Each chunk c left a normalised partial O_c and its lse_c (natural log) in the fp32
// workspace. With M = max_c lse_c: lse = M + ln(sum_c e^(lse_c - M)) and
// O = sum_c e^(lse_c - lse) O_c. Chunks that saw no key (lse_c = -inf) carry no weight;
// a row with no key at all gets O = 0 and lse = -inf. One wave per output row; lanes
// cover head_dim.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.num_merges) return;
  const int lane = threadIdx.x & 63;
  const int* mi = p.merges + 4 * static_cast<int64_t>(item);
  const int out_row = mi[0], ws0 = mi[1], nch = mi[2], stride = mi[3];

  float mx = -INFINITY;
  for (int c = 0; c < nch; ++c) mx = fmaxf(mx, p.ws_lse[ws0 + c * stride]);
  const float mu = mx == -INFINITY ? 0.f : mx;
  constexpr int PER = (D + 63) / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float tot = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int wr = ws0 + c * stride;
    const float lc = p.ws_lse[wr];
    const float w = lc == -INFINITY ? 0.f : expf(lc - mu);
    tot += w;
    const float* src = p.ws_o + static_cast<int64_t>(wr) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + 64 * i;
      if (d < D) acc[i] = fmaf(w, src[d], acc[i]);
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + 64 * i;
    if (d >= D) continue;
    const float ov = acc[i] * inv;
    if (BF16)
      static_cast<uint16_t*>(p.out)[static_cast<int64_t>(out_row) * D + d] = to_bf16_bits(ov);
    else
      static_cast<float*>(p.out)[static_cast<int64_t>(out_row) * D + d] = ov;
  }
  if (lane == 0 && p.lse) p.lse[out_row] = tot > 0.f ? mu + logf(tot) : -INFINITY;
}

template <bool BF16>
hipError_t launch_t(const AttnParams& p, const Launch& l) {
  const dim3 grid((p.num_merges + 3) / 4), block(256);
  switch (p.d) {
    case 16: return launch_kernel(merge_kernel<16, BF16>, grid, block, p, l);
    case 32: return launch_kernel(merge_kernel<32, BF16>, grid, block, p, l);
    case 64: return launch_kernel(merge_kernel<64, BF16>, grid, block, p, l);
    case 128: return launch_kernel(merge_kernel<128, BF16>, grid, block, p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_merge(const AttnParams& p, int dtype, const Launch& l) {
  if (p.num_merges == 0) return hipSuccess;
  return dtype == 1 ? launch_t<true>(p, l) : launch_t<false>(p, l);
}

}  // namespace xattn
