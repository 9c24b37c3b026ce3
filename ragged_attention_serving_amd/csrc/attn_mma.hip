// bf16 attention over query tiles with MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// One workgroup (4 waves) per unit: a request's KV head, up to 128 query rows (32 per
// wave), and a KV range walked in tiles of 64 keys.
//
// Data movement. K and V tiles go straight from HBM to LDS with the 16-byte
// global->LDS loads (no register staging), STAGES tiles deep: while a tile is
// computed the next STAGES-1 are in flight. Both keep their natural row layout
// (key rows of head_dim values) with the 32-byte units of each row XOR-swizzled by
// the row, so that the MFMA operand reads below hit every LDS bank evenly. The page
// indices of the unit's pages are staged in LDS once, so the tile loop issues no
// vector-memory operation other than the tile loads themselves.
//
// Math, per tile and wave:
//   * S^T = K Q^T (keys x the wave's 32 query columns) with Q held in registers as the
//     B operand; a lane owns one query column and 16 of the tile's 64 keys in its
//     accumulators (the other 16 sit in lane ^ 32), so row max and sum need one
//     cross-lane exchange;
//   * online softmax in fp32 (exp2 with log2(e) folded into the scale; the running max
//     only moves when a tile's max exceeds it by more than 2^8, which keeps every
//     weight below 256 and skips nearly all rescales);
//   * O^T += V^T P^T with the probabilities, rounded to bf16, as the B operand taken
//     straight from the accumulators; V^T comes from the LDS transpose reads
//     (ds_read_b64_tr_b16), which hand each lane 4 consecutive keys of one dim, in the
//     key order of the accumulator layout.
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "partition.h"

namespace xattn {

namespace {

constexpr int kBN = 64;  // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <int D>
struct Cfg {
  static constexpr int STAGES = D == 128 ? 2 : 3;
  static constexpr int ROWB = 2 * D;           // bytes per key row
  static constexpr int RPI = 1024 / ROWB;      // key rows per 1 KB load instruction
  static constexpr int LPR = 64 / RPI;         // lanes per key row in a load
  static constexpr int NIW = kBN / RPI / kWaves;  // load instructions per wave per tile (K or V)
  static constexpr int TILE = kBN * ROWB;      // bytes of one K (or V) tile
  // 32-byte unit swizzle: unit c of key row r is stored at unit c ^ swz(r), chosen so
  // that any 8 consecutive rows spread one unit index over the 8 units of a 256-byte
  // bank window
  static __device__ __forceinline__ int swz(int r) { return D == 128 ? (r & 7) : ((r >> 1) & 3); }
};

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt with vmcnt = n (0..63) and the other counters left alone
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// Compiler-only memory barrier around s_barrier: keeps LDS reads and writes on their
// side of the barrier without the full vmcnt(0) drain that __syncthreads implies (the
// tile loads still in flight must stay in flight).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int MASK>
__global__ __launch_bounds__(kThreads, 2) void attn_mma_kernel(AttnParams p) {
  using C = Cfg<D>;
  constexpr int S = C::STAGES;
  constexpr int NKK = D / 16;  // MFMA k-steps for Q.K^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  // one LDS object per (stage, K/V): the compiler then knows which buffer every
  // global->LDS load writes and waits for exactly those before reading a buffer
  __shared__ __attribute__((aligned(1024))) char sk0[C::TILE], sk1[C::TILE], sk2[S == 3 ? C::TILE : 16];
  __shared__ __attribute__((aligned(1024))) char sv0[C::TILE], sv1[C::TILE], sv2[S == 3 ? C::TILE : 16];
  auto kbuf = [&](auto st) -> lds_char* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return (lds_char*)sk0;
    else if constexpr (i == 1) return (lds_char*)sk1;
    else return (lds_char*)sk2;
  };
  auto vbuf = [&](auto st) -> lds_char* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return (lds_char*)sv0;
    else if constexpr (i == 1) return (lds_char*)sv1;
    else return (lds_char*)sv2;
  };

  const int* u = p.units + static_cast<int64_t>(blockIdx.x) * 8;
  const int r = u[0], hk = u[1], row0 = u[2], nrows = u[3], kv0 = u[4], kv1 = u[5], ws_row = u[6];
  const int* rq = p.reqs + 4 * r;
  const int qo_start = rq[0], qo_len = rq[1], kv_len = rq[2], page_base = rq[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int g = p.group;
  const char* kbytes = static_cast<const char*>(p.k);
  const char* vbytes = static_cast<const char*>(p.v);

  // this lane's query column
  const int lrow = 32 * wave + col;
  const bool valid = lrow < nrows;
  const bool wave_active = 32 * wave < nrows;
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

  const int ntiles = kv1 > kv0 ? (kv1 - kv0 + kBN - 1) / kBN : 0;
  const bool paged = p.pages != nullptr;

  // ---- the unit's page indices, staged in LDS once (at most kMmaMaxPages of them)
  __shared__ int spg[kMmaMaxPages];
  auto logical_page = [&](int t) -> int {
    return p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
  };
  const int lp_first = kv1 > kv0 ? logical_page(kv0) : 0;
  if (paged && ntiles > 0) {
    // the partitioner keeps a unit within kMmaMaxPages pages; the clamp only guards LDS
    const int npg = min(logical_page(kv1 - 1) - lp_first + 1, kMmaMaxPages);
    for (int i = tid; i < npg; i += kThreads) spg[i] = p.pages[page_base + lp_first + i];
    __syncthreads();
  }

  // ---- key row ids: lane k of every wave handles key k of a tile (clamped into the range)
  auto page_of = [&](int t) -> int {  // physical page of key t
    const int lp = logical_page(t);
    return paged ? spg[lp - lp_first] : page_base + lp;
  };
  auto row_head = [&](int t, int page) -> int {  // pool (row, head) index of key t
    const int slot = p.page_shift >= 0 ? (t & (p.page_size - 1)) : (t % p.page_size);
    return (page * p.page_size + slot) * p.hkv + hk;
  };
  auto tile_key = [&](int j) -> int { return min(kv0 + j * kBN + lane, kv1 - 1); };

  // ---- global -> LDS loads of one tile into a stage's buffers, from the tile's row ids
  auto issue_tile = [&](auto st, int rh) {
    lds_char* kb = kbuf(st);
    lds_char* vb = vbuf(st);
#pragma unroll
    for (int i = 0; i < C::NIW; ++i) {
      const int n = C::NIW * wave + i;             // 1 KB block of the tile
      const int key = C::RPI * n + lane / C::LPR;  // key row this lane fills
      const int slot16 = lane % C::LPR;            // 16-byte slot within the row
      const int unit = (slot16 >> 1) ^ C::swz(key);
      const int src16 = 2 * unit + (slot16 & 1);   // global 16-byte chunk stored there
      const int rhk = __shfl(rh, key, 64);
      const int64_t off = static_cast<int64_t>(rhk) * C::ROWB + 16 * src16;
      __builtin_amdgcn_global_load_lds(kbytes + off, kb + n * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vbytes + off, vb + n * 1024, 16, 0, 0);
    }
  };

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // ---- one tile: compute tile j from stage ST while tiles j+1 .. j+S-1 are in flight
  int pg_next = 0;
  auto step = [&](auto st, int j) {
    constexpr int ST = decltype(st)::value;
    constexpr int NEXT = (ST + S - 1) % S;  // the stage tile j-1 used
    // this wave's loads for tile j are done once at most the later ones are outstanding
    if constexpr (S == 3) {
      wait_vmcnt(j + 1 < ntiles ? 2 * C::NIW : 0);
    } else {
      wait_vmcnt(0);
    }
    block_barrier();  // every wave's share of tile j is in LDS; every wave is past tile j-1

    // refill the stage tile j-1 used with tile j+S-1 (its page looked up one step ahead)
    if (j + S - 1 < ntiles) {
      const int rh = row_head(tile_key(j + S - 1), pg_next);
      if (j + S < ntiles) pg_next = page_of(tile_key(j + S));
      issue_tile(std::integral_constant<int, NEXT>{}, rh);
    }
    if (!wave_active) return;

    const int t0 = kv0 + j * kBN;
    const lds_char* kb = kbuf(st);
    const lds_char* vb = vbuf(st);

    // S^T = K Q^T for the tile's two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb2][i] = 0.f;
      const int key = 32 * kb2 + col;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        // 16-byte chunk 2kk + half of the key row: unit kk, its half `half`
        const int off = key * C::ROWB + 32 * (kk ^ C::swz(key)) + 16 * half;
        const bf16x8_t a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(kb + off);
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kk], s[kb2], 0, 0, 0);
      }
    }

    // mask: accumulator i of block kb2 holds key t0 + 32kb2 + 8(i/4) + 4half + i%4
    if (__any(t0 + kBN - 1 > lim)) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = t0 + 32 * kb2 + 8 * (i / 4) + 4 * half + (i % 4);
          if (t > lim) s[kb2][i] = -INFINITY;
        }
    }

    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
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
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(s[kb2][8 * jj + e], p.scale_log2, -mu));
          lsum += pv[e];
        }
        const uint4 packed = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                        pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
        pb[2 * kb2 + jj] = __builtin_bit_cast(bf16x8_t, packed);
      }
    }

    // O^T += V^T P^T. k-step st4 covers keys 16st4 + [0, 16): this lane's 8 are
    // 16st4 + 4half + {0..3} and 16st4 + 8 + 4half + {0..3}. The transpose read of a
    // 16-lane group whose lane i addresses key kbase + i/4, dims dbase + 4(i%4) .. +3
    // returns to lane i dim dbase + i of keys kbase .. kbase + 3.
    const int i16 = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int unit = 2 * db + g16;  // 32-byte unit holding dims 32db + 16g16 .. +15
#pragma unroll
      for (int st4 = 0; st4 < 4; ++st4) {
        const int k0 = 16 * st4 + 4 * half + (i16 >> 2);
        const int k1 = k0 + 8;
        const int off0 = k0 * C::ROWB + 32 * (unit ^ C::swz(k0)) + 8 * (i16 & 3);
        const int off1 = k1 * C::ROWB + 32 * (unit ^ C::swz(k1)) + 8 * (i16 & 3);
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) short4_t*>(const_cast<lds_char*>(vb) + off0));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) short4_t*>(const_cast<lds_char*>(vb) + off1));
        const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8), pb[st4], o[db], 0, 0, 0);
      }
    }
  };

  // prologue: tiles 0 .. S-2 in flight; the page of tile S-1 requested
  if (0 < ntiles) {
    const int t = tile_key(0);
    issue_tile(std::integral_constant<int, 0>{}, row_head(t, page_of(t)));
  }
  if constexpr (S == 3) {
    if (1 < ntiles) {
      const int t = tile_key(1);
      issue_tile(std::integral_constant<int, 1>{}, row_head(t, page_of(t)));
    }
  }
  if (S - 1 < ntiles) pg_next = page_of(tile_key(S - 1));

  for (int j = 0; j < ntiles; j += S) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>{}, j + 1);
    if constexpr (S == 3) {
      if (j + 2 < ntiles) step(std::integral_constant<int, 2>{}, j + 2);
    }
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
