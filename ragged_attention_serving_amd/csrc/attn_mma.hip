// bf16 attention over query tiles with MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// One workgroup (NW = 4 or 8 waves) per unit: a request's KV head, up to 32 * NW query
// rows (32 per wave), and a KV range walked in tiles of 64 keys.
//
// Data movement. K and V tiles go straight from HBM to LDS with 16-byte loads that
// write LDS directly (no register staging), in S stages: tile j+S-1 loads while tile j
// computes. S is 3 at head_dim 64 (three stages still fit the three workgroups per CU
// that the registers allow, and keep twice the bytes in flight for short-query units,
// whose steps are short) and 2 at head_dim 128 (a third stage would leave one
// workgroup per CU). When the pools span less than 4 GB the loads are buffer loads whose
// per-lane offsets are 32-bit (the pool base sits in scalar registers); larger pools
// take global loads with 64-bit addresses. Both tiles keep their natural row layout
// (key rows of head_dim values) with the 16-byte chunks of each row XOR-swizzled by the
// row, so that the MFMA operand reads below hit distinct LDS banks. The page indices of
// the unit's pages are staged in LDS once, so the tile loop issues no vector-memory
// operation other than the tile loads themselves. The kernel is instantiated per table
// kind (a page table, or the identity table of packed spans), so its tile loop carries
// only that table's address arithmetic.
//
// Math, per tile and wave:
//   * S^T = K Q^T (keys x the wave's 32 query columns) with Q held in registers as the
//     B operand; a lane owns one query column and 16 of the tile's 64 keys in its
//     accumulators (the other 16 sit in lane ^ 32), so row max and sum need one
//     cross-lane exchange (a VALU swap of the two 32-lane halves);
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

constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <int D, int NW, int BN>
struct Cfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int NKB = BN / 32;          // 32-key blocks per tile
  static constexpr int NST = BN / 16;          // 16-key MFMA k-steps of P V per tile
  static constexpr int ROWB = 2 * D;           // bytes per key row
  static constexpr int RPI = 1024 / ROWB;      // key rows per 1 KB load instruction
  static constexpr int LPR = 64 / RPI;         // lanes per key row in a load
  static constexpr int NIW = BN / RPI / NW;    // load instructions per wave per tile (K or V)
  static_assert(NIW * RPI * NW == BN, "tile split across waves");
  // the per-row table path gives each lane of a wave one key of the tile
  static_assert(BN <= 64, "at most one key per lane in a tile");
  static constexpr int TILE = BN * ROWB;       // bytes of one K (or V) tile
  // 16-byte chunk swizzle: chunk c of key row r is stored in slot c ^ swz(r). With 64
  // banks of 4 bytes (a 256-byte window; a D=128 row fills one, a D=64 row half of one):
  //  * the K operand read has 16 lanes on 16 consecutive rows at one chunk: swz takes 16
  //    distinct values on them (D=128), or 8 distinct values per row parity (D=64);
  //  * a transpose read has 16-lane groups on 4 rows (4-aligned) x 32 bytes, and the two
  //    groups of a half-wave on two adjacent 32-byte units of the same rows: the 4 rows'
  //    swz values differ in bit 2 and above, so the 16 chunks land in 16 distinct slots.
  static __device__ __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

// Compiler-only memory barrier around s_barrier: keeps LDS reads and writes on their
// side of the barrier without the full vmcnt(0) drain that __syncthreads implies.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Lane l and lane l ^ 32 combined through the VALU swap of the 32-lane halves (no LDS
// round trip): the swap leaves each lane its own value in one result and its partner's in
// the other, so a symmetric operation on the two results needs no lane select (and both
// lanes of a pair get the same bits).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// vmcnt(2 * NIW): every load but the last tile's K and V (NIW each per wave) has landed;
// vector-memory loads complete in the order they were issued
template <int NIW>
__device__ __forceinline__ void wait_loads_but_one_tile() {
  static_assert(2 * NIW < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NIW));
}

template <int D, int MASK, int NW, int BN, bool BUF, bool PAGED>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_mma_kernel(AttnParams p) {
  using C = Cfg<D, NW, BN>;
  constexpr int NKB = C::NKB, NST = C::NST;
  constexpr int NKK = D / 16;  // MFMA k-steps for Q.K^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int S = D == 64 ? 3 : 2;  // LDS stages
  // one LDS object per buffer: the compiler then knows which buffer every global->LDS
  // load writes and waits only for those before reading a buffer
  __shared__ __attribute__((aligned(1024))) char sk0[C::TILE], sk1[C::TILE], sk2[S == 3 ? C::TILE : 1];
  __shared__ __attribute__((aligned(1024))) char sv0[C::TILE], sv1[C::TILE], sv2[S == 3 ? C::TILE : 1];

  if (p.unit_count && static_cast<int>(blockIdx.x) >= *p.unit_count) return;  // past this plan's units
  const int* u = p.units + static_cast<int64_t>(blockIdx.x) * 8;
  const int r = u[0], hk = u[1], row0 = u[2], nrows = u[3], kv0 = u[4], kv1 = u[5], ws_row = u[6];
  const int* rq = p.reqs + 4 * r;
  const int qo_start = rq[0], qo_len = rq[1], kv_len = rq[2], page_base = rq[3];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave math scalar
  const int col = lane & 31, half = lane >> 5;
  const int g = p.group;
  const char* kbytes = static_cast<const char*>(p.k);
  const char* vbytes = static_cast<const char*>(p.v);
  // buffer form: no range limit beyond the 32-bit offsets (like the global form)
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.k), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.v), (short)0, -1, 0x00020000);

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

  const int ntiles = kv1 > kv0 ? (kv1 - kv0 + BN - 1) / BN : 0;
  constexpr bool paged = PAGED;  // a page table, or the identity table (no gather)

  // ---- the unit's page indices, staged in LDS once (at most kMmaMaxPages of them)
  __shared__ int spg[kMmaMaxPages];
  auto logical_page = [&](int t) __attribute__((always_inline)) -> int {
    return p.page_shift >= 0 ? (t >> p.page_shift) : (t / p.page_size);
  };
  const int lp_first = kv1 > kv0 ? logical_page(kv0) : 0;
  if (paged && ntiles > 0) {
    // the partitioner keeps a unit within kMmaMaxPages pages; the clamp only guards LDS
    const int npg = min(logical_page(kv1 - 1) - lp_first + 1, kMmaMaxPages);
    for (int i = tid; i < npg; i += C::THREADS) spg[i] = p.pages[page_base + lp_first + i];
    __syncthreads();
  }

  // ---- paged table: pool (row, head) index of key `lane` of tile j (keys past the range
  // clamp to its last key, whose scores are masked)
  auto tile_row_head = [&](int j) __attribute__((always_inline)) -> int {
    const int t = min(kv0 + j * BN + lane, kv1 - 1);
    const int lp = logical_page(t);
    const int page = paged ? spg[lp - lp_first] : page_base + lp;
    const int slot = p.page_shift >= 0 ? (t & (p.page_size - 1)) : (t - lp * p.page_size);
    return (page * p.page_size + slot) * p.hkv + hk;
  };
  // ---- global -> LDS loads of tile j: this wave fills NIW 1 KB blocks of the K tile and
  // the same blocks of the V tile. The byte offsets in the pool (shared by K and V) come
  // from the tile's row ids, the row of key k being held by lane k.
  using Off = typename std::conditional<BUF, uint32_t, int64_t>::type;
  struct TileOffsets {
    Off v[C::NIW];
  };
  // identity table: key t of the request is pool row page_base * page_size + t, so a
  // lane's offsets for tile j are those of tile 0 plus j whole tiles, except in a last
  // tile that runs past the range (its keys clamp to the range's last key)
  TileOffsets id_base;
  const Off id_stride = static_cast<Off>(BN) * p.hkv * C::ROWB;
  auto identity_offsets = [&](int j) __attribute__((always_inline)) -> TileOffsets {
    TileOffsets t;
#pragma unroll
    for (int i = 0; i < C::NIW; ++i) {
      const int n = C::NIW * wave + i;             // 1 KB block of the tile
      const int key = C::RPI * n + lane / C::LPR;  // key row this lane fills
      const int src16 = (lane % C::LPR) ^ C::swz(key);  // global chunk for this slot
      const int row = (page_base * p.page_size + min(kv0 + j * BN + key, kv1 - 1)) * p.hkv + hk;
      t.v[i] = static_cast<Off>(static_cast<uint32_t>(row)) * C::ROWB + 16 * src16;
    }
    return t;
  };
  if (!paged) id_base = identity_offsets(0);
  // paged, buffer form, keys from a page boundary on and pages a multiple of a load's rows:
  // the rows of one 1 KB load lie in one page, so a lane's offset in a whole tile is that
  // page's start (its index read from LDS) plus a constant of the unit
  const bool pg_whole = BUF && paged && p.page_shift >= 0 && (BN & (p.page_size - 1)) == 0 &&
                        (p.page_size % C::RPI) == 0 && (kv0 & (p.page_size - 1)) == 0;
  const uint32_t pg_bytes = static_cast<uint32_t>(p.page_size * p.hkv * C::ROWB);
  uint32_t pg_const[C::NIW];
#pragma unroll
  for (int i = 0; i < C::NIW; ++i) {
    const int key = C::RPI * (C::NIW * wave + i) + lane / C::LPR;
    const int src16 = (lane % C::LPR) ^ C::swz(key);
    pg_const[i] = static_cast<uint32_t>((((key & (p.page_size - 1)) * p.hkv + hk) * C::ROWB) + 16 * src16);
  }
  auto tile_offsets = [&](int j) __attribute__((always_inline)) -> TileOffsets {
    TileOffsets t;
    if (!paged) {
      if (kv0 + (j + 1) * BN > kv1) return identity_offsets(j);
      const Off add = id_stride * j;
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) t.v[i] = id_base.v[i] + add;
      return t;
    }
    if (pg_whole && kv0 + (j + 1) * BN <= kv1) {
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) {
        const int key = C::RPI * (C::NIW * wave + i) + lane / C::LPR;
        const uint32_t page = static_cast<uint32_t>(spg[(j * BN + key) >> p.page_shift]);
        t.v[i] = static_cast<Off>(page * pg_bytes + pg_const[i]);
      }
      return t;
    }
    const int rh = tile_row_head(j);
#pragma unroll
    for (int i = 0; i < C::NIW; ++i) {
      const int n = C::NIW * wave + i;
      const int key = C::RPI * n + lane / C::LPR;
      const int src16 = (lane % C::LPR) ^ C::swz(key);
      t.v[i] = static_cast<Off>(static_cast<uint32_t>(__shfl(rh, key, 64))) * C::ROWB + 16 * src16;
    }
    return t;
  };
  // `which`: 0 loads from the K pool, 1 from the V pool
  auto issue_one = [&](auto which, lds_char* dst, const TileOffsets& t, int i) __attribute__((always_inline)) {
    // (every address is a variable of its own: with template-dependent expressions in
    // the builtins' arguments, the host compilation pass silently drops the kernel's
    // launch stub)
    const int n = C::NIW * wave + i;
    lds_char* d = dst + n * 1024;
    if constexpr (BUF) {
      const uint32_t off = t.v[i];
      const __amdgpu_buffer_rsrc_t rs = decltype(which)::value ? rsv : rsk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, off, 0, 0, 0);
    } else {
      const char* g = (decltype(which)::value ? vbytes : kbytes) + t.v[i];
      __builtin_amdgcn_global_load_lds(g, d, 16, 0, 0);
    }
  };
  using PoolK = std::integral_constant<int, 0>;
  using PoolV = std::integral_constant<int, 1>;
  auto issue = [&](auto which, lds_char* dst, int j) __attribute__((always_inline)) {
    const TileOffsets t = tile_offsets(j);
#pragma unroll
    for (int i = 0; i < C::NIW; ++i) issue_one(which, dst, t, i);
  };

  // ---- per-lane LDS read offsets (bytes within a buffer), fixed for the unit.
  // K operand of block kb, k-step kk: row 32kb + col, chunk 2kk + half; swz depends only
  // on col, so block kb adds 32 rows (an immediate).
  int koff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = col * C::ROWB + 16 * ((2 * kk + half) ^ C::swz(col));
  // V^T operand of block db, k-step st4: this lane's transpose reads address key rows
  // k0 = 16st4 + 4half + i16/4 and k0 + 8 at dims 32db + 16g16 + 4(i16%4); swz of those
  // rows does not depend on st4, so st4 adds 16 rows (an immediate).
  const int i16 = lane & 15, g16 = (lane >> 4) & 1;
  int voff[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const int k0 = 4 * half + (i16 >> 2) + 8 * h8;
      const int c16 = 4 * db + 2 * g16 + ((i16 & 3) >> 1);
      voff[db][h8] = k0 * C::ROWB + 16 * (c16 ^ C::swz(k0)) + 8 * (i16 & 1);
    }

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  // running max (log2 units) and this lane's partial row sum, both in fp32; the max only
  // changes in the rare rescale, which also updates what each tile reads of it: the
  // exponent offset (minus the max, or 0 while no key has been seen) and the raw-score
  // level above which a tile moves the max
  float m = -INFINITY, lsum = 0.f;
  float neg_m = 0.f, raw_level = -INFINITY;
  const float inv_scale = 1.f / p.scale_log2;

  // max of the raw scores over a lane's query column: its 32 accumulators, then the 32 in
  // lane ^ 32 (IEEE maximum: -inf for masked keys, no quieting step on its inputs)
  auto column_max = [&](const f32x16_t (&s)[NKB]) __attribute__((always_inline)) -> float {
    float mx = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, s[0][i]);
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, s[kb][i]);
    return pair_max(mx);
  };

  // ---- prologue: tile 0 in LDS (and, with three stages, tile 1 on its way)
  if (ntiles > 0) {
    issue(PoolK{}, (lds_char*)sk0, 0);
    issue(PoolV{}, (lds_char*)sv0, 0);
  }
  if constexpr (S == 3) {
    if (ntiles > 0) {
      const int t1 = ntiles > 1 ? 1 : 0;  // a one-tile unit reloads tile 0: no load behind a branch
      issue(PoolK{}, (lds_char*)sk1, t1);
      issue(PoolV{}, (lds_char*)sv1, t1);
      wait_loads_but_one_tile<C::NIW>();
    } else {
      wait_all_loads();
    }
  } else {
    wait_all_loads();
  }
  block_barrier();

  // ---- step j: tile j is in buffer j % S. Load tile j+S-1 into buffer (j+S-1) % S, the
  // one tile j-1 used (every wave is past tile j-1), compute tile j, then wait for tile
  // j+1 (with three stages the loads just issued stay in flight) and meet at the barrier.
  auto step = [&](auto par, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr int N = (P + S - 1) % S;  // buffer of the tile loaded in this step
    lds_char* kcur = (lds_char*)(P == 0 ? sk0 : P == 1 ? sk1 : sk2);
    lds_char* vcur = (lds_char*)(P == 0 ? sv0 : P == 1 ? sv1 : sv2);
    lds_char* knext = (lds_char*)(N == 0 ? sk0 : N == 1 ? sk1 : sk2);
    lds_char* vnext = (lds_char*)(N == 0 ? sv0 : N == 1 ? sv1 : sv2);
    // the last steps reload their own tile into the free buffer (an L2 hit that nothing
    // reads), so that no load sits behind a branch
    const TileOffsets nxt = tile_offsets(j + S - 1 < ntiles ? j + S - 1 : j);
    if (!wave_active) {
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) issue_one(PoolK{}, knext, nxt, i);
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) issue_one(PoolV{}, vnext, nxt, i);
    }
    if (wave_active) {
      // S^T = K Q^T for the tile's 32-key blocks; accumulator i of block kb holds key
      // 32kb + 8(i/4) + 4half + i%4 of the tile. All K fragments of the tile are read
      // first, so their LDS latencies overlap; the blocks' MFMA chains then interleave.
      bf16x8_t ka[NKB][NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          ka[kb][kk] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
              kcur + koff[kk] + 32 * kb * C::ROWB);
      f32x16_t sc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
      // the next tile's loads go out one at a time between the MFMAs, so that no wave
      // waits at a full address queue before it can compute
      static_assert(NKK % (2 * C::NIW) == 0 || (2 * C::NIW) % NKK == 0, "load spread");
      constexpr int PER_KK = (2 * C::NIW + NKK - 1) / NKK;  // loads after each k-step
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][kk], qb[kk], sc[kb], 0, 0, 0);
#pragma unroll
        for (int x = 0; x < PER_KK; ++x) {
          const int i = kk * PER_KK + x;
          if (i < C::NIW) issue_one(PoolK{}, knext, nxt, i);
          else if (i < 2 * C::NIW) issue_one(PoolV{}, vnext, nxt, i - C::NIW);
        }
      }

      // V^T fragments for P V, read now so that they arrive while the softmax runs.
      // k-step st4 covers keys 16st4 + [0, 16): this lane's 8 are 16st4 + 4half + {0..3}
      // and 16st4 + 8 + 4half + {0..3}. The transpose read of a 16-lane group whose lane
      // i addresses key kbase + i/4, dims dbase + 4(i%4) .. +3 returns to lane i dim
      // dbase + i of keys kbase .. kbase + 3.
      bf16x8_t va[NDB][NST];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int st4 = 0; st4 < NST; ++st4) {
          const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) short4_t*>(vcur + voff[db][0] + 16 * st4 * C::ROWB));
          const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) short4_t*>(vcur + voff[db][1] + 16 * st4 * C::ROWB));
          const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          va[db][st4] = __builtin_bit_cast(bf16x8_t, a8);
        }

      // keys past the last one this query sees: key 32kb + 8(i/4) + 4half + i%4 is
      // visible iff 32kb + 8(i/4) + i%4 <= lim - t0 - 4half (a compare with a constant)
      const int t0 = kv0 + j * BN;
      if (__any(t0 + BN - 1 > lim)) {
        const int d = lim - t0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb + 8 * (i / 4) + (i % 4) > d) sc[kb][i] = -INFINITY;
      }
      const float mx = column_max(sc);
      if (__any(mx > raw_level)) {
        const float mn = fmaxf(m, mx * p.scale_log2);
        const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        m = mn;
        neg_m = mn == -INFINITY ? 0.f : -mn;
        raw_level = (mn + kRescaleSlack) * inv_scale;
      }

      // probabilities, row sums, and the bf16 B operands for P V (k-step = 16 keys)
      bf16x8_t pb[NST];
#pragma unroll
      for (int b = 0; b < NST; ++b) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(sc[b / 2][8 * (b % 2) + e], p.scale_log2, neg_m));
          lsum += pv[e];
        }
        const uint4 packed = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                        pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
        pb[b] = __builtin_bit_cast(bf16x8_t, packed);
      }

      // O^T += V^T P^T
#pragma unroll
      for (int st4 = 0; st4 < NST; ++st4)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][st4], pb[st4], o[db], 0, 0, 0);
    }
    if constexpr (S == 3) wait_loads_but_one_tile<C::NIW>();
    else wait_all_loads();
    block_barrier();
  };
  for (int j = 0; j < ntiles; j += S) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>{}, j + 1);
    if constexpr (S == 3)
      if (j + 2 < ntiles) step(std::integral_constant<int, 2>{}, j + 2);
  }
  if constexpr (S == 3) wait_all_loads();  // no load may land in LDS after the workgroup ends

  // ---- finish: O / l and lse; accumulator i of block db holds dim 32db + 8(i/4) + 4half + i%4
  const float lt = pair_sum(lsum);
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

template <int D, int NW, int BN, bool BUF, bool PAGED>
hipError_t launch_dwbp(const AttnParams& p, const Launch& l) {
  const dim3 grid(p.num_units), block(64 * NW);
  switch (p.mask) {
    case 0: return launch_kernel(attn_mma_kernel<D, 0, NW, BN, BUF, PAGED>, grid, block, p, l);
    case 1: return launch_kernel(attn_mma_kernel<D, 1, NW, BN, BUF, PAGED>, grid, block, p, l);
    case 2: return launch_kernel(attn_mma_kernel<D, 2, NW, BN, BUF, PAGED>, grid, block, p, l);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int NW, int BN, bool BUF>
hipError_t launch_dwb(const AttnParams& p, const Launch& l) {
  if (p.pages != nullptr) return launch_dwbp<D, NW, BN, BUF, true>(p, l);
  return launch_dwbp<D, NW, BN, BUF, false>(p, l);
}

// buffer loads (32-bit offsets) when both pools span less than 4 GB
template <int D, int NW, int BN>
hipError_t launch_dw(const AttnParams& p, const Launch& l) {
  if (buffer_loads_fit(p)) return launch_dwb<D, NW, BN, true>(p, l);
  return launch_dwb<D, NW, BN, false>(p, l);
}

constexpr int kTileKeys = 64;  // keys per K/V tile

template <int D>
hipError_t launch_d(const AttnParams& p, const Launch& l) {
  if (p.tile_rows == 128) return launch_dw<D, 4, kTileKeys>(p, l);
  if (p.tile_rows == 256) return launch_dw<D, 8, 64>(p, l);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_mma(const AttnParams& p, const Launch& l) {
  if (p.num_units == 0) return hipSuccess;
  switch (p.d) {
    case 64: return launch_d<64>(p, l);
    case 128: return launch_d<128>(p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xattn
