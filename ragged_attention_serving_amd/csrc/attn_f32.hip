// fp32 attention kernel: exact fp32 arithmetic for fp32 inputs, every mask mode.
//
// One workgroup per unit (a request's KV head, up to 4 query rows, a KV chunk of at
// most 1024 keys). Three phases, each a plain data-parallel loop:
//   1. scores s[row][t] = scale * q_row . k_t for the chunk's keys, into LDS
//      (masked keys get -inf);
//   2. per row (one wave each): m = max s, p = exp(s - m), l = sum p;
//   3. O[row][d] = sum_t p[row][t] v_t[d] / l, threads over (row, d) so that each
//      value row is read with consecutive lanes on consecutive dims.
// The whole chunk's scores fit in LDS, so no online rescaling is needed.
#include "device.h"
#include "kernels.h"
#include "partition.h"

namespace xattn {

namespace {

constexpr int kRows = kF32Rows;
constexpr int kMaxChunk = kF32MaxChunk;

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnParams p) {
  __shared__ float sQ[kRows][D];
  __shared__ float sS[kRows][kMaxChunk];
  __shared__ float sM[kRows], sL[kRows];

  if (p.unit_count && static_cast<int>(blockIdx.x) >= *p.unit_count) return;  // past this plan's units
  const int* u = p.units + static_cast<int64_t>(blockIdx.x) * 8;
  const int r = u[0], hk = u[1], row0 = u[2], nrows = u[3], kv0 = u[4], kv1 = u[5], ws_row = u[6];
  const int* rq = p.reqs + 4 * r;
  const int qo_start = rq[0], qo_len = rq[1], kv_len = rq[2], page_base = rq[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = p.group;
  const float* q = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k);
  const float* vp = static_cast<const float*>(p.v);
  const int n = kv1 - kv0;

  for (int i = tid; i < kRows * D; i += 256) {
    const int rr = i / D, d = i % D;
    float x = 0.f;
    if (rr < nrows) {
      const int row = row0 + rr;
      const int qi = row / g, h = hk * g + row % g;
      x = q[(static_cast<int64_t>(qo_start + qi) * p.hq + h) * D + d];
    }
    sQ[rr][d] = x;
  }
  int lim[kRows];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) {
    const int row = row0 + rr;
    lim[rr] = rr < nrows ? min(last_visible(p.mask, p.block, qo_len, kv_len, row / g), kv1 - 1) : -1;
  }
  __syncthreads();

  // phase 1: scores
  for (int t = tid; t < n; t += 256) {
    const int key = kv0 + t;
    const float* kr = kp + kv_offset(kv_row(p, page_base, key), p.hkv, hk, D);
    float acc[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) acc[rr] = 0.f;
    for (int d = 0; d < D; d += 4) {
      const float4 kk = *reinterpret_cast<const float4*>(kr + d);
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) {
        acc[rr] = fmaf(sQ[rr][d + 0], kk.x, acc[rr]);
        acc[rr] = fmaf(sQ[rr][d + 1], kk.y, acc[rr]);
        acc[rr] = fmaf(sQ[rr][d + 2], kk.z, acc[rr]);
        acc[rr] = fmaf(sQ[rr][d + 3], kk.w, acc[rr]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) sS[rr][t] = key <= lim[rr] ? acc[rr] * p.scale : -INFINITY;
  }
  __syncthreads();

  // phase 2: max, exponentials and sum, one wave per row
  {
    const int rr = wave;
    float mx = -INFINITY;
    for (int t = lane; t < n; t += 64) mx = fmaxf(mx, sS[rr][t]);
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, m));
    float sum = 0.f;
    for (int t = lane; t < n; t += 64) {
      const float e = mx == -INFINITY ? 0.f : expf(sS[rr][t] - mx);
      sS[rr][t] = e;
      sum += e;
    }
    for (int m = 32; m >= 1; m >>= 1) sum += shfl_xor_f(sum, m);
    if (lane == 0) {
      sM[rr] = mx;
      sL[rr] = sum;
    }
  }
  __syncthreads();

  // phase 3: weighted sum of values
  for (int i = tid; i < kRows * D; i += 256) {
    const int rr = i / D, d = i % D;
    if (rr >= nrows) continue;
    float acc = 0.f;
    for (int t = 0; t < n; ++t) {
      const float w = sS[rr][t];
      if (w != 0.f) acc = fmaf(w, vp[kv_offset(kv_row(p, page_base, kv0 + t), p.hkv, hk, D) + d], acc);
    }
    const float l = sL[rr];
    const float o = l > 0.f ? acc / l : 0.f;
    const float lse = l > 0.f ? sM[rr] + logf(l) : -INFINITY;
    const int row = row0 + rr;
    if (ws_row >= 0) {
      p.ws_o[static_cast<int64_t>(ws_row + rr) * D + d] = o;
      if (d == 0) p.ws_lse[ws_row + rr] = lse;
    } else {
      const int64_t orow = static_cast<int64_t>(qo_start + row / g) * p.hq + hk * g + row % g;
      static_cast<float*>(p.out)[orow * D + d] = o;
      if (d == 0 && p.lse) p.lse[orow] = lse;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, const Launch& l) {
  if (p.num_units == 0) return hipSuccess;
  const dim3 grid(p.num_units), block(256);
  switch (p.d) {
    case 16: return launch_kernel(attn_f32_kernel<16>, grid, block, p, l);
    case 32: return launch_kernel(attn_f32_kernel<32>, grid, block, p, l);
    case 64: return launch_kernel(attn_f32_kernel<64>, grid, block, p, l);
    case 128: return launch_kernel(attn_f32_kernel<128>, grid, block, p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xattn
