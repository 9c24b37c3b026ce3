// bf16 decode attention: a few query rows per KV head, bound by HBM bandwidth.
//
// One workgroup (4 waves) per unit: a request's KV head, its R query rows (query
// tokens x the query heads that share the KV head, so each K/V row read from HBM
// serves every grouped head), and a chunk of keys. Eight lanes cover one key's
// head_dim (16 bytes each for D=64, 32 for D=128), so a wave reads 8 keys per step as
// whole 128-byte segments; the 4 waves interleave steps so the workgroup streams
// consecutive keys. Per key: q.k by packed bf16 dot products with fp32 accumulation,
// summed over the 8 lanes with DPP. Each lane keeps an online softmax (running max,
// sum and its slice of O in fp32) for the keys of its lane group; the 32 partial
// states of the workgroup are merged at the end (shuffles within a wave, LDS across
// waves). The unit's page indices are staged in LDS first, so each step's address
// needs no global load, and K/V are read with non-temporal loads.
#include "device.h"
#include "kernels.h"
#include "partition.h"

namespace xattn {

namespace {

// 16-byte load of K/V data that is read exactly once: a non-temporal (streaming) load,
// so the pass over the cache does not displace anything that is reused
__device__ __forceinline__ uint4 load16(const uint4* ptr) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr)));
}

constexpr int kWaves = 4;
constexpr int kLanesPerKey = 8;
constexpr int kKeysPerStep = 64 / kLanesPerKey;  // keys per wave per step
constexpr int kSteps = 4;  // steps per loop iteration

template <int D, int R>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnParams p) {
  constexpr int CPL = D / (8 * kLanesPerKey);  // 16-byte chunks per lane per key
  constexpr int DPL = CPL * 8;                 // dims per lane
  constexpr int kKeysPerIter = kWaves * kSteps * kKeysPerStep;
  __shared__ float sM[kWaves][R], sL[kWaves][R];
  __shared__ float sO[kWaves][R][D];
  __shared__ int spg[kDecMaxPages];

  if (p.unit_count && static_cast<int>(blockIdx.x) >= *p.unit_count) return;  // past this plan's units
  const int* u = p.units + static_cast<int64_t>(blockIdx.x) * 8;
  const int r = u[0], hk = u[1], row0 = u[2], nrows = u[3], kv0 = u[4], kv1 = u[5], ws_row = u[6];
  const int* rq = p.reqs + 4 * r;
  const int qo_start = rq[0], qo_len = rq[1], kv_len = rq[2], page_base = rq[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kslot = lane / kLanesPerKey, csub = lane % kLanesPerKey;
  const int g = p.group;
  const uint16_t* qp = static_cast<const uint16_t*>(p.q);
  const uint16_t* kp = static_cast<const uint16_t*>(p.k);
  const uint16_t* vp = static_cast<const uint16_t*>(p.v);

  // query rows: lane holds chunks csub + 8*i of each row
  uint4 qv[R][CPL];
  int lim[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int row = row0 + rr;
    if (rr < nrows) {
      const int qi = row / g, h = hk * g + row % g;
      const uint4* qr = reinterpret_cast<const uint4*>(qp + (static_cast<int64_t>(qo_start + qi) * p.hq + h) * D);
#pragma unroll
      for (int i = 0; i < CPL; ++i) qv[rr][i] = qr[csub + kLanesPerKey * i];
      lim[rr] = min(last_visible(p.mask, p.block, qo_len, kv_len, qi), kv1 - 1);
    } else {
#pragma unroll
      for (int i = 0; i < CPL; ++i) qv[rr][i] = make_uint4(0, 0, 0, 0);
      lim[rr] = -1;
    }
  }

  // the unit's page indices, staged in LDS once (at most kDecMaxPages of them)
  const bool paged = p.pages != nullptr;
  auto logical_page = [&](int t) -> int {
    return p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
  };
  const int lp_first = kv1 > kv0 ? logical_page(kv0) : 0;
  if (paged && kv1 > kv0) {
    // the partitioner keeps a unit within kDecMaxPages pages; the clamp only guards LDS
    const int npg = min(logical_page(kv1 - 1) - lp_first + 1, kDecMaxPages);
    for (int i = tid; i < npg; i += 256) spg[i] = p.pages[page_base + lp_first + i];
    __syncthreads();
  }
  auto key_offset = [&](int t) -> int64_t {  // element offset of (key t, kv head hk, dim 0)
    const int lp = logical_page(t);
    const int page = paged ? spg[lp - lp_first] : page_base + lp;
    const int slot = p.page_shift >= 0 ? (t & (p.page_size - 1)) : (t - lp * p.page_size);
    return (static_cast<int64_t>(page) * p.page_size + slot) * p.hkv * D + static_cast<int64_t>(hk) * D;
  };

  float m[R], l[R], o[R][DPL];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    m[rr] = -INFINITY;
    l[rr] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[rr][j] = 0.f;
  }

  for (int base = kv0; base < kv1; base += kKeysPerIter) {
    uint4 kr[kSteps][CPL], vr[kSteps][CPL];
    int key[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int t = base + (s * kWaves + wave) * kKeysPerStep + kslot;
      key[s] = t;
      if (t < kv1) {
        const int64_t off = key_offset(t);
        const uint4* k4 = reinterpret_cast<const uint4*>(kp + off);
        const uint4* v4 = reinterpret_cast<const uint4*>(vp + off);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          kr[s][i] = load16(k4 + csub + kLanesPerKey * i);
          vr[s][i] = load16(v4 + csub + kLanesPerKey * i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          kr[s][i] = make_uint4(0, 0, 0, 0);
          vr[s][i] = make_uint4(0, 0, 0, 0);
        }
      }
    }

    // scores in log2 units: s = scale*log2(e) * q.k, -inf where masked
    float sc[kSteps][R];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          acc = dot2_bf16(qv[rr][i].x, kr[s][i].x, acc);
          acc = dot2_bf16(qv[rr][i].y, kr[s][i].y, acc);
          acc = dot2_bf16(qv[rr][i].z, kr[s][i].z, acc);
          acc = dot2_bf16(qv[rr][i].w, kr[s][i].w, acc);
        }
        acc = sum8(acc);
        sc[s][rr] = key[s] <= lim[rr] ? acc * p.scale_log2 : -INFINITY;
      }
    }

    // online softmax update, then accumulate p * v
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      float mx = sc[0][rr];
#pragma unroll
      for (int s = 1; s < kSteps; ++s) mx = fmaxf(mx, sc[s][rr]);
      const float mn = fmaxf(m[rr], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[rr] - mu);
      m[rr] = mn;
      l[rr] *= alpha;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[rr][j] *= alpha;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const float pw = fast_exp2(sc[s][rr] - mu);
        l[rr] += pw;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const uint4 vv = vr[s][i];
          o[rr][8 * i + 0] = fmaf(pw, bf16_lo(vv.x), o[rr][8 * i + 0]);
          o[rr][8 * i + 1] = fmaf(pw, bf16_hi(vv.x), o[rr][8 * i + 1]);
          o[rr][8 * i + 2] = fmaf(pw, bf16_lo(vv.y), o[rr][8 * i + 2]);
          o[rr][8 * i + 3] = fmaf(pw, bf16_hi(vv.y), o[rr][8 * i + 3]);
          o[rr][8 * i + 4] = fmaf(pw, bf16_lo(vv.z), o[rr][8 * i + 4]);
          o[rr][8 * i + 5] = fmaf(pw, bf16_hi(vv.z), o[rr][8 * i + 5]);
          o[rr][8 * i + 6] = fmaf(pw, bf16_lo(vv.w), o[rr][8 * i + 6]);
          o[rr][8 * i + 7] = fmaf(pw, bf16_hi(vv.w), o[rr][8 * i + 7]);
        }
      }
    }
  }

  // merge the 8 key slots of the wave (lanes csub, csub+8, ..., csub+56)
#pragma unroll
  for (int x = 8; x < 64; x <<= 1) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const float mo = shfl_xor_f(m[rr], x);
      const float lo = shfl_xor_f(l[rr], x);
      const float mn = fmaxf(m[rr], mo);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float a = fast_exp2(m[rr] - mu), b = fast_exp2(mo - mu);
      l[rr] = l[rr] * a + lo * b;
      m[rr] = mn;
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const float oo = shfl_xor_f(o[rr][j], x);
        o[rr][j] = o[rr][j] * a + oo * b;
      }
    }
  }
  if (kslot == 0) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      if (csub == 0) {
        sM[wave][rr] = m[rr];
        sL[wave][rr] = l[rr];
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) sO[wave][rr][8 * (csub + kLanesPerKey * i) + e] = o[rr][8 * i + e];
    }
  }
  __syncthreads();

  // merge the 4 waves and write one (row, dim) per thread
  for (int idx = tid; idx < R * D; idx += 256) {
    const int rr = idx / D, d = idx % D;
    if (rr >= nrows) continue;
    float mx = sM[0][rr];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sM[w][rr]);
    const float mu = mx == -INFINITY ? 0.f : mx;
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = fast_exp2(sM[w][rr] - mu);
      lt += a * sL[w][rr];
      ot += a * sO[w][rr][d];
    }
    const float ov = lt > 0.f ? ot / lt : 0.f;
    const float lse = lt > 0.f ? (mu + __log2f(lt)) * kLn2 : -INFINITY;
    const int row = row0 + rr;
    if (ws_row >= 0) {
      p.ws_o[static_cast<int64_t>(ws_row + rr) * D + d] = ov;
      if (d == 0) p.ws_lse[ws_row + rr] = lse;
    } else {
      const int64_t orow = static_cast<int64_t>(qo_start + row / g) * p.hq + hk * g + row % g;
      static_cast<uint16_t*>(p.out)[orow * D + d] = to_bf16_bits(ov);
      if (d == 0 && p.lse) p.lse[orow] = lse;
    }
  }
}

template <int D>
hipError_t launch_rows(const AttnParams& p, int rows, const Launch& l) {
  const dim3 grid(p.num_units), block(256);
  switch (rows) {
    case 1: return launch_kernel(attn_decode_kernel<D, 1>, grid, block, p, l);
    case 2: return launch_kernel(attn_decode_kernel<D, 2>, grid, block, p, l);
    case 4: return launch_kernel(attn_decode_kernel<D, 4>, grid, block, p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_decode(const AttnParams& p, int rows, const Launch& l) {
  if (p.num_units == 0) return hipSuccess;
  switch (p.d) {
    case 64: return launch_rows<64>(p, rows, l);
    case 128: return launch_rows<128>(p, rows, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xattn
