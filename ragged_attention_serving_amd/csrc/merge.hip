// Split-KV merge: rebuild an output row from the partial results of its KV chunks.
//
// Each chunk c left a normalised partial O_c and its lse_c (natural log) in the fp32
// workspace. With M = max_c lse_c: lse = M + ln(sum_c e^(lse_c - M)) and
// O = sum_c e^(lse_c - lse) O_c. Chunks that saw no key (lse_c = -inf) carry no weight;
// a row with no key at all gets O = 0 and lse = -inf.
//
// D/4 lanes per output row (4 dims each, 16-byte loads), so a wave merges 256/D rows.
// The chunks are taken four at a time with a running maximum: the four lse values and
// the four partial rows of a group are loaded together, so a row costs one round trip
// to memory per group of chunks instead of one per chunk.
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kGroup = 4;  // chunks loaded together

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  constexpr int L = D / 4;        // lanes per row
  constexpr int RPW = 64 / L;     // rows per wave
  const int lane = threadIdx.x & 63;
  const int item = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / L;
  if (item >= (p.merge_count ? *p.merge_count : p.num_merges)) return;
  const int sub = lane % L;       // dims 4sub .. 4sub+3
  const int4 mi = *reinterpret_cast<const int4*>(p.merges + 4 * static_cast<int64_t>(item));
  const int out_row = mi.x, ws0 = mi.y, nch = mi.z, stride = mi.w;

  float m = -INFINITY, tot = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nch; c0 += kGroup) {
    float lc[kGroup];
    float4 oc[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      lc[g] = -INFINITY;
      oc[g] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + g < nch) {
        const int64_t wr = ws0 + static_cast<int64_t>(c0 + g) * stride;
        lc[g] = p.ws_lse[wr];
        oc[g] = *reinterpret_cast<const float4*>(p.ws_o + wr * D + 4 * sub);
      }
    }
    float mn = m;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) mn = fmaxf(mn, lc[g]);
    if (mn == -INFINITY) continue;  // no chunk so far saw a key
    const float r = expf(m - mn);   // m = -inf gives 0, and acc and tot are still 0
    tot *= r;
    acc.x *= r, acc.y *= r, acc.z *= r, acc.w *= r;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const float w = expf(lc[g] - mn);  // lse_c = -inf gives weight 0
      tot += w;
      acc.x = fmaf(w, oc[g].x, acc.x);
      acc.y = fmaf(w, oc[g].y, acc.y);
      acc.z = fmaf(w, oc[g].z, acc.z);
      acc.w = fmaf(w, oc[g].w, acc.w);
    }
    m = mn;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int64_t base = static_cast<int64_t>(out_row) * D + 4 * sub;
  if (BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + base) =
        make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + base) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (sub == 0 && p.lse) p.lse[out_row] = tot > 0.f ? m + logf(tot) : -INFINITY;
}

template <bool BF16>
hipError_t launch_t(const AttnParams& p, const Launch& l) {
  const int rows_per_block = 4 * (256 / p.d);  // 4 waves of 256/D rows
  const dim3 grid((p.num_merges + rows_per_block - 1) / rows_per_block), block(256);
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
