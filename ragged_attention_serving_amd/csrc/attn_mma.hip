// bf16 attention over query tiles with MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// One workgroup (4 waves) per unit: a request's KV head, up to 128 query rows (32 per
// wave), and a KV range walked in tiles of 64 keys. Per tile:
//   * the workgroup stages K [64][D] and V transposed [D][64] in LDS (double
//     buffered; the next tile's global loads are in flight while this one computes);
//   * each wave computes S^T = K Q^T (keys x its 32 query columns) with Q held in
//     registers as the B operand, so a lane owns one query column and 16 of the
//     tile's keys in its accumulators, and the other 16 sit in lane ^ 32: the row
//     max and sum need one cross-lane exchange;
//   * online softmax in fp32 (exp2 with log2(e) folded into the scale; the running
//     max is only raised when a tile's max exceeds it by more than 2^8, which keeps
//     every weight below 256 and skips nearly all rescales);
//   * O^T += V^T P^T with the probabilities, rounded to bf16, as the B operand
//     straight from the accumulator registers (the key order of each k-step follows
//     the accumulator layout, and V^T is read from LDS in that same order).
#include "device.h"
#include "kernels.h"

namespace xattn {

namespace {

constexpr int kBN = 64;      // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D>
struct Smem {
  static constexpr int KS = D + 8;    // K row stride (elements): 16-byte reads conflict free
  static constexpr int VS = kBN + 4;  // V^T row stride (elements): 8-byte reads conflict free
  uint16_t k[2][kBN * KS];
  uint16_t v[2][D * VS];
};

template <int D, int MASK>
__global__ __launch_bounds__(kThreads, 2) void attn_mma_kernel(AttnParams p) {
  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  constexpr int NKK = D / 16;                 // MFMA k-steps for Q.K^T
  constexpr int NDB = D / 32;                 // 32-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per key row
  constexpr int NKC = kBN * CPR / kThreads;   // K chunks per thread per tile
  constexpr int NVG = (kBN / 4) * CPR;        // 4-key x 8-dim V groups per tile
  static_assert(NKC * kThreads == kBN * CPR, "K tile split");
  static_assert(NVG <= kThreads, "V tile split");
  __shared__ Smem<D> sm;

  const int* u = p.units + static_cast<int64_t>(blockIdx.x) * 8;
  const int r = u[0], hk = u[1], row0 = u[2], nrows = u[3], kv0 = u[4], kv1 = u[5], ws_row = u[6];
  const int* rq = p.reqs + 4 * r;
  const int qo_start = rq[0], qo_len = rq[1], kv_len = rq[2], page_base = rq[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int g = p.group;
  const uint16_t* kp = static_cast<const uint16_t*>(p.k);
  const uint16_t* vp = static_cast<const uint16_t*>(p.v);

  // this lane's query column
  const int lrow = 32 * wave + col;  // row within the unit
  const bool valid = lrow < nrows;
  const int row = row0 + lrow;
  const int qi = row / g, head = hk * g + row % g;
  bf16x8_t qb[NKK];
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (static_cast<int64_t>(qo_start + qi) * p.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (valid) x = *reinterpret_cast<const uint4*>(qr + 16 * kk + 8 * half);
      qb[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  const int lim = valid ? min(last_visible(MASK, p.block, qo_len, kv_len, qi), kv1 - 1) : kv1 - 1;

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // ---- staging: global -> registers -> LDS
  uint4 kreg[NKC];
  uint4 vreg[4];
  const int vcol = tid / 16, vkey4 = tid % 16;  // V group of this thread (if tid < NVG)

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int idx = tid + kThreads * i;
      const int key = idx / CPR, c = idx % CPR;
      const int t = t0 + key;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (t < kv1)
        kreg[i] = *reinterpret_cast<const uint4*>(kp + kv_offset(kv_row(p, page_base, t), p.hkv, hk, D) + 8 * c);
    }
    if (tid < NVG) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * vkey4 + i;
        vreg[i] = make_uint4(0, 0, 0, 0);
        if (t < kv1)
          vreg[i] = *reinterpret_cast<const uint4*>(vp + kv_offset(kv_row(p, page_base, t), p.hkv, hk, D) + 8 * vcol);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int idx = tid + kThreads * i;
      const int key = idx / CPR, c = idx % CPR;
      *reinterpret_cast<uint4*>(&sm.k[buf][key * KS + 8 * c]) = kreg[i];
    }
    if (tid < NVG) {
      const uint32_t a[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t b[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t c2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t d2[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 2w (low halves) and 2w+1 (high halves) of keys 4*vkey4 + 0..3
        const uint32_t lo01 = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(d2[w], c2[w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(d2[w], c2[w], 0x07060302u);
        *reinterpret_cast<uint2*>(&sm.v[buf][(8 * vcol + 2 * w) * VS + 4 * vkey4]) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(&sm.v[buf][(8 * vcol + 2 * w + 1) * VS + 4 * vkey4]) = make_uint2(hi01, hi23);
      }
    }
  };

  const int ntiles = kv1 > kv0 ? (kv1 - kv0 + kBN - 1) / kBN : 0;
  if (ntiles > 0) {
    load_tile(kv0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int t0 = kv0 + j * kBN;
    if (j + 1 < ntiles) load_tile(t0 + kBN);

    // S^T = K Q^T for the tile's two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&sm.k[buf][(32 * kb + col) * KS + 16 * kk + 8 * half]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kk], s[kb], 0, 0, 0);
      }
    }

    // mask: accumulator i of block kb holds key t0 + 32kb + 8(i/4) + 4half + i%4
    if (__any(t0 + kBN - 1 > lim)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = t0 + 32 * kb + 8 * (i / 4) + 4 * half + (i % 4);
          if (t > lim) s[kb][i] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mxs = mx * p.scale_log2;
    if (__any(mxs > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mxs);
      const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m = mn;
    }
    const float mu = m == -INFINITY ? 0.f : m;

    // probabilities, row sums, and the bf16 B operands for P V (k-step = 16 keys)
    bf16x8_t pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(s[kb][8 * jj + e], p.scale_log2, -mu));
          lsum += pv[e];
        }
        uint4 packed = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
        pb[2 * kb + jj] = __builtin_bit_cast(bf16x8_t, packed);
      }
    }

    // O^T += V^T P^T; k-step (kb, jj) covers keys 32kb + 16jj + [0, 16): this lane's
    // 8 are 32kb + 16jj + 4half + {0..3} and the same + 8
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vrow = &sm.v[buf][(32 * db + col) * VS + 4 * half];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kofs = 16 * st;  // 32kb + 16jj with st = 2kb + jj
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kofs);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + kofs + 8);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[db], 0, 0, 0);
      }
    }

    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- finish: O / l and lse; accumulator i of block db holds dim 32db + 8(i/4) + 4half + i%4
  const float lt = lsum + shfl_xor_f(lsum, 32);
  if (!valid) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  if (ws_row >= 0) {
    float* dst = p.ws_o + static_cast<int64_t>(ws_row + lrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * half;
        *reinterpret_cast<float4*>(dst + d) =
            make_float4(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv);
      }
    if (half == 0) p.ws_lse[ws_row + lrow] = lse;
  } else {
    const int64_t orow = static_cast<int64_t>(qo_start + qi) * p.hq + head;
    uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * half;
        *reinterpret_cast<uint2*>(dst + d) =
            make_uint2(pack_bf16x2(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv),
                       pack_bf16x2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv));
      }
    if (half == 0 && p.lse) p.lse[orow] = lse;
  }
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(p.num_units), block(kThreads);
  switch (p.mask) {
    case 0: hipLaunchKernelGGL((attn_mma_kernel<D, 0>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((attn_mma_kernel<D, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((attn_mma_kernel<D, 2>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mma(const AttnParams& p, hipStream_t stream) {
  if (p.num_units == 0) return hipSuccess;
  switch (p.d) {
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xattn
