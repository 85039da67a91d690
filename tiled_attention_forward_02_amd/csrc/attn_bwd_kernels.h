// attn_bwd_kernels.h - device code of the attention backward (dQ, dK, dV) for
// gfx950 (CDNA4): the tile layout, the dQ kernel, the key-side kernel and
// their launch. Included by attn_bwd.hip (d = 32 to 128, built with the
// MFMA accumulators held in VGPRs) and attn_bwd256.hip (d = 256, built with
// the accumulators free to live in AGPRs); see attn_bwd.hip for what the
// kernels compute.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "common.h"
#include "mi_attn.h"

namespace mi_attn {

struct BwdArgs {
  const void *q, *k, *v, *o, *d_o;
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;
  int BH, Nq, Nk, nq, nk, nw;
  bool dq_pp;  // dQ by the ping-pong kernel (d = 128): nq counts its 256-row workgroups
  float c, scale;
  hipStream_t stream;
};

// The d = 256 launch (both kernels), in attn_bwd256.hip.
hipError_t launch_bwd_d256(const BwdArgs& a, bool causal, bool f16);

}  // namespace mi_attn

namespace {

using namespace mi_attn;


// Query rows (dQ) or keys (dK/dV) per workgroup: 32 a wave, four waves a
// workgroup and two workgroups a CU, or at d = 128 without the causal mask,
// on big grids with long rows, eight waves, one workgroup a CU. Eight waves
// halve the HBM -> LDS staging per FLOP (each streamed tile serves twice the
// rows): +2.9% on B=16 H=16 N=4096 d=128 and +0.7% on B=4 H=16 N=2048, but
// -0.8% on B=8 H=16 N=1024, where the loop is too short to hide the start
// and end of a workgroup that has its CU to itself (measured interleaved,
// bit-identical outputs). Causal, the bigger workgroups lose (-0.5% on
// B=1 H=32 N=16384 d=128, -6.6% on B=8 H=16 N=2048 d=64; the last row
// blocks of a causal grid carry the most work; in the dK/dV kernel alone
// -2.2% on the first and -3.8% on B=4 H=16 N=2048), and so they do at d = 32
// (-3.8%), 64 (-2.8% on B=16 H=16 N=4096, -3.2% on B=8 H=16 N=2048) and 96
// (-2.0%).
constexpr int kBlockRows = 32 * kWaves;  // with four waves; the size checks use it

// Workgroups per CU the register allocation must allow: two (two waves a
// SIMD) below d = 256. At d = 256 one: a key-side wave holds K and V
// fragments (128 registers) and two 128-register accumulators, which only
// fit in one wave's 512 (accumulators in AGPRs), so those kernels run one
// wave a SIMD.
template <int D, int NW>
constexpr int kBwdMinBlocks = D == 256 ? 1 : 8 / NW;

// Rows per streamed tile (keys in the dQ kernel, queries in the dK/dV
// kernel).
template <int D>
constexpr int kTileRows = D <= 64 ? 64 : 32;

// Head dimension of the LDS tile layout: d = 96 tiles are laid out as
// d = 128 ones, 12 of 16 chunks per row staged and read (as in the forward).
template <int D>
constexpr int kLayoutD = D == 96 ? 128 : D;

// A tile of BR rows of a [*, D] tensor in LDS: one row-major copy that
// serves both 16-byte row reads (an MFMA A operand of rows) and transposing
// reads (lds_read_tr16: an A operand of columns). Row pitch P elements is an
// odd multiple of 64 bytes, and the 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 2) & 3). With the LDS's 64 banks of 4 bytes:
//  * a transposing-read pass (32 lanes) covers 4 consecutive rows x one
//    64-byte group of 4 chunks; the swizzle permutes chunks only within a
//    group, and the rows' groups start 64 bytes apart mod 256: no conflict;
//  * a row-read pass (16 lanes, 16 bytes each) covers 16 rows at one
//    chunk; the pitch alone would put them in 4 bank groups, the swizzle
//    spreads them over all 16.
// The tile is loaded by LDS DMA, the swizzle applied through each lane's
// source offset; it takes SPAN bytes of LDS (a multiple of 1024). Each lane
// keeps its DMA offsets, two row-read bases (the chunk pair's low bits XOR
// the swizzle take two values) and two transposing-read offsets (rows +0
// and +8 of a slice).
template <int D, int BR, int WAVES>
struct SwzTile {
  static constexpr int DL = kLayoutD<D>;
  static constexpr int P = DL % 64 == 32 ? DL : DL + 32;  // row pitch, elements
  static constexpr int SLOTS = P / 8, CPR = DL / 8;
  static constexpr int NINSTR = (BR * SLOTS + 63) / 64;
  static constexpr int NW = (NINSTR + WAVES - 1) / WAVES;  // per wave, at most
  static constexpr int SPAN = NINSTR * 1024;
  static constexpr uint32_t kNoFetch = 0x80000000u;  // + row0 * D * 2 < 2^31
  static_assert((P * 2) % 128 == 64, "pitch: an odd multiple of 64 bytes");
  uint32_t off[NW];
  uint32_t rrd[2], trd[2];
  static __device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
  __device__ __forceinline__ SwzTile(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int slot = 64 * (wave + WAVES * i) + lane;
      const int row = slot / SLOTS, pc = slot % SLOTS;
      const int c = pc ^ swz(row);  // logical chunk held by physical chunk pc
      off[i] = row < BR && pc < CPR && c < D / 8 ? (uint32_t)(row * D + 8 * c) * 2 : kNoFetch;
    }
    const int col = lane & 31, h = lane >> 5, g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      rrd[e] = (uint32_t)(col * P + 8 * ((2 * e + h) ^ swz(col))) * 2;
      trd[e] = (uint32_t)((4 * (g >> 1) + (s >> 2) + 8 * e) * P +
                          8 * ((2 * (g & 1) + ((s & 3) >> 1)) ^ (((g >> 1) + 2 * e) & 3)) +
                          4 * (s & 1)) * 2;
    }
  }
  __device__ __forceinline__ void issue(rsrc_t r, lds_char* tile, int wave, int row0) const {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int u = wave + WAVES * i;
      if (u < NINSTR) load16_lds(r, tile + 1024 * u, off[i] + (uint32_t)row0 * D * 2);
    }
  }
  // A operand of rows 32 blk + lane % 32, k-elements 16 j + 8 h .. +7.
  template <typename V8>
  __device__ __forceinline__ V8 rows(const char* tile, int blk, int j) const {
    return *reinterpret_cast<const V8*>(tile + rrd[j & 1] + (32 * blk * P + 32 * (j >> 1)) * 2);
  }
  // A operand of columns col0 .. col0 + 31 over rows row0 .. row0 + 15 (a
  // 16-row slice, row0 a multiple of 16), rows in slice_pos order: the lane
  // layout of tr_lane_off, with each lane's chunk moved by the swizzle.
  template <typename V8>
  __device__ __forceinline__ V8 cols(const char* tile, int row0, int col0) const {
    const char* q = tile + (row0 * P + col0) * 2;
    const u32x2 lo = lds_read_tr16(q + trd[0]), hi = lds_read_tr16(q + trd[1]);
    return __builtin_bit_cast(V8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
};

// 2^(s*c - l2), the weight of a score s given the row's lse in log2 units.
__device__ __forceinline__ float weight(float s, float c, float l2) {
  return __builtin_amdgcn_exp2f(fmaf(s, c, -l2));
}

// The forward's lse of a row, in log2 units; +inf for a row that sees no key
// (lse = -inf) or lies past the end, so that its weights are all 0.
__device__ __forceinline__ float lse_log2(float lse, bool valid) {
  return (valid && lse != -INFINITY) ? lse * kLog2e : INFINITY;
}

// ------------------------------------------------------------- dQ kernel --

template <typename E, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, (kBwdMinBlocks<D, NW>)) void attn_bwd_dq_kernel(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const E* __restrict__ O, const float* __restrict__ LSE, const E* __restrict__ dO,
    E* __restrict__ dQ, float* __restrict__ Delta, int BH, int Nq, int Nk, int nq, float c,
    float dq_scale) {
  constexpr int BN = kTileRows<D>;
  using G = SwzTile<D, BN, NW>;
  constexpr int NKB = BN / 32;
  // Stage: K | V (K is read both as rows and as columns).
  constexpr int V_OFF = G::SPAN;
  constexpr int STAGE = 2 * G::SPAN;
  typedef typename Elem<E>::v8 v8;
  typedef typename Elem<E>::v4 v4;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  int bh, qt;
  map_block(blockIdx.x, BH, nq, CAUSAL, bh, qt);
  const int q0 = qt * 32 * NW;
  const int qw = q0 + 32 * wave;
  const int qi = qw + col;
  const int off = Nk - Nq;  // query i sits at key position i + off

  const size_t qhead = (size_t)bh * (size_t)Nq * D;
  const size_t khead = (size_t)bh * (size_t)Nk * D;
  const uint32_t q_bytes = (uint32_t)Nq * D * 2;
  const uint32_t k_bytes = (uint32_t)Nk * D * 2;
  const rsrc_t rk = make_rsrc(K + khead, k_bytes);
  const rsrc_t rv = make_rsrc(V + khead, k_bytes);

  // Q^T and dO^T fragments (B operands, a query per lane), and D_i from this
  // lane's half of the row of dO * O, both halves combined.
  v8 qf[D / 16], df[D / 16];
  float dpart = 0.f;
  {
    const rsrc_t rq = make_rsrc(Q + qhead, q_bytes);
    const rsrc_t rdo = make_rsrc(dO + qhead, q_bytes);
    const rsrc_t ro = make_rsrc(O + qhead, q_bytes);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t at = (uint32_t)(qi * D + 16 * s + 8 * half) * 2;
      qf[s] = __builtin_bit_cast(v8, load16(rq, at));
      df[s] = __builtin_bit_cast(v8, load16(rdo, at));
      const v8 o8 = __builtin_bit_cast(v8, load16(ro, at));
#pragma unroll
      for (int j = 0; j < 8; ++j) dpart = fmaf((float)df[s][j], (float)o8[j], dpart);
    }
  }
  const float delta = swap_halves_add(dpart);
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
  const float l2 = lse_log2(
      __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, qi * 4, 0, 0)), qi < Nq);
  if (half == 0) {
    const rsrc_t rd = make_rsrc(Delta + (size_t)bh * Nq, (uint32_t)Nq * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(delta), rd, qi * 4, 0, 0);
  }

  const int kv_end = CAUSAL ? min(Nk, q0 + 32 * NW + off) : Nk;
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int wave_kv_end = CAUSAL ? min(Nk, qw + 32 + off) : Nk;

  // The key tile from k0 into a stage, by DMA.
  const G tile(wave, lane);
  char* const lds = smem;
  lds_char* const lds3 = to_lds(smem);
  auto stage_tile = [&](auto stage_c, int k0) __attribute__((always_inline)) {
    constexpr uint32_t base = decltype(stage_c)::value * STAGE;
    tile.issue(rk, lds3 + base, wave, k0);
    tile.issue(rv, lds3 + base + V_OFF, wave, k0);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  // -D in every register of a block: the first dP^T MFMA of each tile reads
  // it as its accumulator input, so dP^T - D comes out of the chain with no
  // subtraction per element. Its 16 registers stay live throughout; at
  // d = 32 they would cost the fourth wave per SIMD, so d = 32 subtracts.
  constexpr bool kNegD = D >= 64;
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = kNegD ? -delta : 0.f;

  auto step = [&](int t, auto stage_c) __attribute__((always_inline)) {
    constexpr uint32_t base = decltype(stage_c)::value * STAGE;
    const int k0 = t * BN;
    const bool has_next = t + 1 < nt;
    if (has_next) stage_tile(std::integral_constant<int, decltype(stage_c)::value ^ 1>{}, k0 + BN);

    if (k0 < wave_kv_end) {
      // S^T = K Q^T and dP^T = V dO^T (less D), 32 keys per accumulator.
      f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const v8 ka = tile.template rows<v8>(lds + base, kb, j);
          const v8 va = tile.template rows<v8>(lds + base + V_OFF, kb, j);
          sacc[kb] = Elem<E>::mfma(ka, qf[j], j == 0 ? f32x16{} : sacc[kb]);
          pacc[kb] = Elem<E>::mfma(va, df[j], j == 0 ? (kNegD ? negd : f32x16{}) : pacc[kb]);
        }
      }
      // P, with 0 for keys past Nk and (causal) keys after the query.
      float p[NKB][16];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) p[kb][i] = weight(sacc[kb][i], c, l2);
      if ((k0 + BN > Nk) || (CAUSAL && k0 + BN - 1 > qw + off)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
            if (key >= Nk || (CAUSAL && key > qi + off)) p[kb][i] = 0.f;
          }
      }
      // dS^T = P^T (dP^T - D), rounded: the B operand of dQ^T += K^T dS^T.
      v8 dsb[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dsb[kb][i >> 3][i & 7] = (E)(p[kb][i] * (kNegD ? pacc[kb][i] : pacc[kb][i] - delta));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const v8 a = tile.template cols<v8>(lds + base, 32 * kb + 16 * sg, 32 * db);
            acc[db] = Elem<E>::mfma(a, dsb[kb][sg], acc[db]);
          }
    }

    // The next tile lands in LDS with no instruction of this wave writing it:
    // wait for its loads before the barrier.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (nt > 0) {
    stage_tile(std::integral_constant<int, 0>{}, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }

  // dQ = scale * acc; rows past Nq are dropped by the range check.
  const rsrc_t rdq = make_rsrc(dQ + qhead, q_bytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)(acc[db][4 * r + e] * dq_scale);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), rdq,
                                            (int)((qi * D + 32 * db + 8 * r + 4 * half) * 2),
                                            0, 0);
    }
}

// --------------------------------------------- dQ ping-pong kernel (d = 128) --
// The eight-wave dQ shape at d = 128: 256 queries a workgroup, 32 a wave, one
// workgroup a CU; waves w and w + 4 share a SIMD.
// Each wave alternates an MFMA phase M(t) (dQ^T += K^T dS^T of key tile
// t-1, then S^T = K Q^T and dP^T = V dO^T of tile t) and a VALU phase X(t)
// (P and dS of tile t), with a workgroup barrier after each; waves 4-7 run
// one phase behind waves 0-3, so on every SIMD one wave's MFMAs run beside
// the other's VALU work (in step, both waves of a SIMD issued MFMAs at the
// same time and then both their VALU work).
//
// A key tile's K is read from the phase that computes its S until the one
// that adds its dQ, four phases, so the tiles go round a ring of four LDS
// stages. Tile t + 2 is loaded during M(t): K by waves 0-3, V by waves 4-7,
// three DMA instructions a wave (each part is padded from ten instructions
// to twelve, the last two writing zeros past the rows, so no wave
// branches). Operands are read three MFMAs ahead. With the causal mask the
// workgroup walks the key tiles up to its last row's; a wave whose rows see
// none of a tile's keys (or only some) gets P = 0 for those keys, so its dQ
// MFMAs add exact zeros and the MFMA sequence keeps no branch.
template <typename E, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_pp_kernel(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const E* __restrict__ O, const float* __restrict__ LSE, const E* __restrict__ dO,
    E* __restrict__ dQ, float* __restrict__ Delta, int BH, int Nq, int Nk, int nq, float c,
    float dq_scale) {
  constexpr int D = 128, NW = 8, BN = 32, NST = 4, PD = 3;
  using G = SwzTile<D, BN, NW>;  // layout and reads of a tile part
  using GD = SwzTile<D, BN, 4>;  // its DMA, dealt to four waves
  static_assert(GD::NINSTR == 10 && GD::NW == 3, "three DMA instructions a wave per part");
  constexpr int PART = 12 * 1024;  // ten instructions of rows, two of padding
  constexpr int V_OFF = PART, STAGE = 2 * PART;
  typedef typename Elem<E>::v8 v8;
  typedef typename Elem<E>::v4 v4;
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const bool late = wave >= 4;
  const int dwave = wave & 3;
  int bh, qt;
  map_block(blockIdx.x, BH, nq, CAUSAL, bh, qt);
  const int q0 = qt * 32 * NW;
  const int qw = q0 + 32 * wave;  // first query of this wave
  const int qi = qw + col;
  const int off = Nk - Nq;  // query i sees key j iff j <= i + off (causal)

  const size_t qhead = (size_t)bh * (size_t)Nq * D;
  const size_t khead = (size_t)bh * (size_t)Nk * D;
  const uint32_t q_bytes = (uint32_t)Nq * D * 2;
  const uint32_t k_bytes = (uint32_t)Nk * D * 2;
  // This wave's DMA part: K (waves 0-3) or V (waves 4-7).
  const rsrc_t rpart = make_rsrc((late ? V : K) + khead, k_bytes);
  const uint32_t part_off = late ? (uint32_t)V_OFF : 0u;

  // Q^T and dO^T fragments (B operands, a query per lane), and D_i from this
  // lane's half of the row of dO * O, both halves combined.
  v8 qf[D / 16], df[D / 16];
  float dpart = 0.f;
  {
    const rsrc_t rq = make_rsrc(Q + qhead, q_bytes);
    const rsrc_t rdo = make_rsrc(dO + qhead, q_bytes);
    const rsrc_t ro = make_rsrc(O + qhead, q_bytes);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t at = (uint32_t)(qi * D + 16 * s + 8 * half) * 2;
      qf[s] = __builtin_bit_cast(v8, load16(rq, at));
      df[s] = __builtin_bit_cast(v8, load16(rdo, at));
      const v8 o8 = __builtin_bit_cast(v8, load16(ro, at));
#pragma unroll
      for (int j = 0; j < 8; ++j) dpart = fmaf((float)df[s][j], (float)o8[j], dpart);
    }
  }
  const float delta = swap_halves_add(dpart);
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
  const float l2 = lse_log2(
      __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, qi * 4, 0, 0)), qi < Nq);
  if (half == 0) {
    const rsrc_t rd = make_rsrc(Delta + (size_t)bh * Nq, (uint32_t)Nq * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(delta), rd, qi * 4, 0, 0);
  }
  const int kv_end = CAUSAL ? min(Nk, q0 + 32 * NW + off) : Nk;
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;

  const G tile(wave, lane);
  const GD dtile(dwave, lane);
  const char* const lds = smem;
  lds_char* const lds3 = to_lds(smem);
  auto dma = [&](uint32_t base, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < GD::NW; ++i)
      load16_lds(rpart, lds3 + base + part_off + 1024 * (dwave + 4 * i),
                 dtile.off[i] + (uint32_t)k0 * D * 2);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  // -D in every register of a block: the accumulator input of each tile's
  // first dP^T MFMA, so dP^T - D needs no subtraction per element.
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -delta;
  // dS of the last tile (the B operand of dQ), and the first operands of the
  // next MFMA phase, read at the end of the VALU phase.
  v8 dsb[2];
  v8 pre[PD];

  // MFMA k of an MFMA phase: k < 8 adds tile t-1's dQ (16-key slice k / 4,
  // output columns 32 (k % 4)); k >= 8 adds step (k - 8) / 2 of tile t's S
  // (even) or dP (odd).
  auto operand = [&](uint32_t bprev, uint32_t bcur, int k) __attribute__((always_inline)) {
    if (k < 8) return tile.template cols<v8>(lds + bprev, 16 * (k / 4), 32 * (k % 4));
    const int j = (k - 8) / 2;
    return tile.template rows<v8>(lds + bcur + ((k & 1) ? V_OFF : 0), 0, j);
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // One tile t in stage st = t % 4 (phases 2t and 2t + 1 for waves 0-3,
  // 2t + 1 and 2t + 2 for waves 4-7).
  auto body = [&](int t, auto st_c, auto first_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    constexpr bool first = decltype(first_c)::value;
    constexpr uint32_t bcur = st * STAGE, bprev = ((st + 3) % NST) * STAGE;
    constexpr uint32_t bload = ((st + 2) % NST) * STAGE;
    constexpr int k_begin = first ? 8 : 0;
    f32x16 sacc, pacc;  // S^T and dP^T - D of tile t
    v8 f[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) f[i] = first ? operand(bprev, bcur, k_begin + i) : pre[i];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = k_begin; k < 24; ++k) {
      if (k + PD < 24) f[(k - k_begin + PD) % (PD + 1)] = operand(bprev, bcur, k + PD);
      const v8 a = f[(k - k_begin) % (PD + 1)];
      if (k < 8) {
        acc[k % 4] = Elem<E>::mfma(a, dsb[k / 4], acc[k % 4]);
      } else {
        const int j = (k - 8) / 2;
        if (k & 1)
          pacc = Elem<E>::mfma(a, df[j], j == 0 ? negd : pacc);
        else
          sacc = Elem<E>::mfma(a, qf[j], j == 0 ? f32x16{} : sacc);
      }
      // Tile t + 2 (zeros past Nk) into the stage tile t - 2 left, after the
      // first S step.
      if (k == 9) {
        __builtin_amdgcn_sched_barrier(0);
        dma(bload, (t + 2) * BN);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    barrier();
    // P = 2^(s c - lse), 0 for keys past Nk (and, causal, past the row's
    // last visible key), and dS^T = P^T (dP^T - D).
    const int k0 = t * BN;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = weight(sacc[i], c, l2);
    if ((k0 + BN > Nk) || (CAUSAL && k0 + BN - 1 > qw + off)) {
      const int lim = CAUSAL ? min(Nk - 1, qi + off) : Nk - 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key > lim) p[i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dsb[i >> 3][i & 7] = (E)(p[i] * pacc[i]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PD; ++i) pre[i] = operand(bcur, 0, i);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA
    barrier();
  };

  // Prologue: tiles 0 and 1 (K by waves 0-3, V by waves 4-7); waves 4-7
  // then pass one extra barrier, which puts them one phase behind.
  if (nt > 0) {
    dma(0, 0);
    dma(STAGE, BN);
  }
  __builtin_amdgcn_s_waitcnt(0);
  barrier();
  if (late) barrier();
  using no = std::false_type;
  if (nt > 0) body(0, std::integral_constant<int, 0>{}, std::true_type{});
  for (int t = 1; t < nt; t += 4) {
    body(t, std::integral_constant<int, 1>{}, no{});
    if (t + 1 < nt) body(t + 1, std::integral_constant<int, 2>{}, no{});
    if (t + 2 < nt) body(t + 2, std::integral_constant<int, 3>{}, no{});
    if (t + 3 < nt) body(t + 3, std::integral_constant<int, 0>{}, no{});
  }
  // dQ of the last tile; waves 0-3 then pass the barrier that evens the
  // counts.
  if (nt > 0) {
    const uint32_t blast = (uint32_t)((nt - 1) % NST) * STAGE;
    v8 f[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) f[i] = pre[i];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k + PD < 8) f[(k + PD) % (PD + 1)] = operand(blast, 0, k + PD);
      acc[k % 4] = Elem<E>::mfma(f[k % (PD + 1)], dsb[k / 4], acc[k % 4]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  if (!late) barrier();

  // dQ = scale * acc; rows past Nq are dropped by the range check.
  const rsrc_t rdq = make_rsrc(dQ + qhead, q_bytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)(acc[db][4 * r + e] * dq_scale);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), rdq,
                                            (int)((qi * D + 32 * db + 8 * r + 4 * half) * 2),
                                            0, 0);
    }
}

// ---------------------------------------------------------- dK/dV kernel --

// One pass accumulates both dK and dV: the K and V fragments and the two
// accumulators fit two waves per SIMD at every head dimension (248 VGPRs at
// d = 128, 254 with the causal mask, no spills).

// LDS stage of the key-side kernel:
//   Q (rows: S = Q K^T; columns: dK) | dO (rows: dP; columns: dV) | lse | D
template <int D, int NW>
struct KeyStage {
  static constexpr int BQ = kTileRows<D>;
  using G = SwzTile<D, BQ, NW>;
  static constexpr int DO_OFF = G::SPAN;
  static constexpr int L_OFF = 2 * G::SPAN;
  static constexpr int D_OFF = L_OFF + BQ * 4;
  static constexpr int BYTES = D_OFF + BQ * 4;
  static_assert(BYTES % 16 == 0 && L_OFF % 16 == 0, "16-byte aligned LDS tiles");
};

// PART: 0 accumulates both gradients in one pass; at d = 256 two passes (1:
// dV only, 2: dK only) each hold one accumulator.
template <typename E, int D, bool CAUSAL, int NW, int PART = 0>
__global__ __launch_bounds__(64 * NW, (kBwdMinBlocks<D, NW>)) void attn_bwd_kv_kernel(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const float* __restrict__ LSE, const E* __restrict__ dO, const float* __restrict__ Delta,
    E* __restrict__ dK, E* __restrict__ dV, int BH, int Nq, int Nk, int nk, float c,
    float dk_scale) {
  using S_ = KeyStage<D, NW>;
  using G = typename S_::G;
  constexpr int BQ = S_::BQ;
  constexpr int NQB = BQ / 32;
  constexpr int STAGE = S_::BYTES;
  typedef typename Elem<E>::v8 v8;
  typedef typename Elem<E>::v4 v4;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  int bh, kt;
  map_block(blockIdx.x, BH, nk, CAUSAL, bh, kt);
  // Causal: key tile 0 sees the most queries; map_block deals the last index
  // first, so number the key tiles from the end.
  if (CAUSAL) kt = nk - 1 - kt;
  const int k0 = kt * 32 * NW;
  const int kw = k0 + 32 * wave;  // first key of this wave
  const int kj = kw + col;        // this lane's key
  const int off = Nk - Nq;        // query i sees key j iff j <= i + off (causal)

  const size_t qhead = (size_t)bh * (size_t)Nq * D;
  const size_t khead = (size_t)bh * (size_t)Nk * D;
  const uint32_t q_bytes = (uint32_t)Nq * D * 2;
  const uint32_t k_bytes = (uint32_t)Nk * D * 2;
  const rsrc_t rq = make_rsrc(Q + qhead, q_bytes);
  const rsrc_t rdo = make_rsrc(dO + qhead, q_bytes);
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
  const rsrc_t rd = make_rsrc(Delta + (size_t)bh * Nq, (uint32_t)Nq * 4);

  // K^T and V^T fragments (B operands, a key per lane); zero past Nk.
  v8 kf[D / 16], vf[D / 16];
  {
    const rsrc_t rk = make_rsrc(K + khead, k_bytes);
    const rsrc_t rv = make_rsrc(V + khead, k_bytes);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t at = (uint32_t)(kj * D + 16 * s + 8 * half) * 2;
      kf[s] = __builtin_bit_cast(v8, load16(rk, at));
      if constexpr (PART != 1) vf[s] = __builtin_bit_cast(v8, load16(rv, at));
    }
  }

  // Query tiles that can see a key of this workgroup: i >= k0 - off.
  const int q_begin = CAUSAL ? max(0, k0 - off) : 0;
  const int qt0 = q_begin / BQ;
  const int nt = q_begin < Nq ? (Nq + BQ - 1) / BQ - qt0 : 0;

  // The query tile from q0 into a stage, by DMA; its lse and D (threads
  // tid < BQ) through registers, kept raw until written to LDS at the end of
  // the step: using them at once would wait for every load in flight, the
  // tile's own included.
  const G tile(wave, lane);
  char* const lds = smem;
  lds_char* const lds3 = to_lds(smem);
  uint32_t lraw = 0, draw = 0;
  bool lvalid = false;
  auto gload = [&](auto stage_c, int q0) __attribute__((always_inline)) {
    constexpr uint32_t base = decltype(stage_c)::value * STAGE;
    tile.issue(rq, lds3 + base, wave, q0);
    tile.issue(rdo, lds3 + base + S_::DO_OFF, wave, q0);
    if (tid < BQ) {
      const int qrow = q0 + tid;
      lvalid = qrow < Nq;
      lraw = __builtin_amdgcn_raw_buffer_load_b32(rl, qrow * 4, 0, 0);
      draw = __builtin_amdgcn_raw_buffer_load_b32(rd, qrow * 4, 0, 0);
    }
  };
  // D goes in negated: it starts the dP accumulator, so dP - D comes out of
  // the MFMA chain with no subtraction per element.
  auto lds_store = [&](auto stage_c) __attribute__((always_inline)) {
    constexpr uint32_t base = decltype(stage_c)::value * STAGE;
    if (tid < BQ) {
      *reinterpret_cast<float*>(lds + base + S_::L_OFF + tid * 4) =
          lse_log2(__uint_as_float(lraw), lvalid);
      *reinterpret_cast<uint32_t*>(lds + base + S_::D_OFF + tid * 4) = draw ^ 0x80000000u;
    }
  };
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  auto step = [&](int t, auto stage_c) __attribute__((always_inline)) {
    constexpr uint32_t base = decltype(stage_c)::value * STAGE;
    const int q0 = (qt0 + t) * BQ;
    const bool has_next = t + 1 < nt;
    if (has_next) gload(std::integral_constant<int, decltype(stage_c)::value ^ 1>{}, q0 + BQ);

    // Some query of the tile sees a key of this wave.
    if (!CAUSAL || q0 + BQ - 1 + off >= kw) {
      // S = Q K^T (and dP - D = dO V^T - D for dK, the chain started at -D),
      // 32 queries per accumulator. Register i of block qb holds query
      // q0 + 32qb + 8(i/4) + 4h + i%4: its lse and -D come four at a time
      // from LDS.
      f32x16 sacc[NQB], pacc[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        sacc[qb] = f32x16{};
        if constexpr (PART != 1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 32 * qb + 8 * r + 4 * half;
            const f32x4 nd4 = *reinterpret_cast<const f32x4*>(lds + base + S_::D_OFF + row * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) pacc[qb][4 * r + e] = nd4[e];
          }
        }
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          sacc[qb] = Elem<E>::mfma(tile.template rows<v8>(lds + base, qb, j), kf[j], sacc[qb]);
          if constexpr (PART != 1)
            pacc[qb] = Elem<E>::mfma(tile.template rows<v8>(lds + base + S_::DO_OFF, qb, j),
                                     vf[j], pacc[qb]);
        }
      }
      const bool masked = CAUSAL && q0 + off < kw + 31;
      v8 pb[NQB][2], dsb[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 32 * qb + 8 * r + 4 * half;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lds + base + S_::L_OFF + row * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * r + e;
            float p = weight(sacc[qb][i], c, l4[e]);
            if (masked && kj > q0 + row + e + off) p = 0.f;
            if constexpr (PART != 2) pb[qb][i >> 3][i & 7] = (E)p;
            if constexpr (PART != 1) dsb[qb][i >> 3][i & 7] = (E)(p * pacc[qb][i]);
          }
        }
      // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per MFMA.
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            if constexpr (PART != 2)
              dvacc[db] = Elem<E>::mfma(
                  tile.template cols<v8>(lds + base + S_::DO_OFF, 32 * qb + 16 * sg, 32 * db),
                  pb[qb][sg], dvacc[db]);
            if constexpr (PART != 1)
              dkacc[db] = Elem<E>::mfma(
                  tile.template cols<v8>(lds + base, 32 * qb + 16 * sg, 32 * db), dsb[qb][sg],
                  dkacc[db]);
          }
    }

    if (has_next) lds_store(std::integral_constant<int, decltype(stage_c)::value ^ 1>{});
    // The next tile lands in LDS with no instruction of this wave writing it:
    // wait for its loads before the barrier.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (nt > 0) {
    gload(std::integral_constant<int, 0>{}, qt0 * BQ);
    lds_store(std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }

  // dK = scale * dK^T acc, dV = dV^T acc; keys past Nk are dropped.
  const rsrc_t rdk = make_rsrc(dK + khead, k_bytes);
  const rsrc_t rdv = make_rsrc(dV + khead, k_bytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int at = (kj * D + 32 * db + 8 * r + 4 * half) * 2;
      v4 x4;
      if constexpr (PART != 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x4[e] = (E)(dkacc[db][4 * r + e] * dk_scale);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x4), rdk, at, 0, 0);
      }
      if constexpr (PART != 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x4[e] = (E)dvacc[db][4 * r + e];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x4), rdv, at, 0, 0);
      }
    }
}

// ------------------------------------------------------------- launch --

template <typename E, int D, bool CAUSAL, int NW>
hipError_t launch_bwd(const BwdArgs& a) {
  const E* q = static_cast<const E*>(a.q);
  const E* k = static_cast<const E*>(a.k);
  const E* v = static_cast<const E*>(a.v);
  const E* o = static_cast<const E*>(a.o);
  const E* d_o = static_cast<const E*>(a.d_o);
  E* dq = static_cast<E*>(a.dq);
  E* dk = static_cast<E*>(a.dk);
  E* dv = static_cast<E*>(a.dv);
  const float* lse = a.lse;
  float* delta = a.delta;
  int BH = a.BH, Nq = a.Nq, Nk = a.Nk, nq = a.nq, nk = a.nk;
  float c = a.c, scale = a.scale;
  // dQ (and D) first: the key-side kernel reads D.
  if (nq > 0) {
    void* args[] = {&q, &k, &v, &o, &lse, &d_o, &dq, &delta, &BH, &Nq, &Nk, &nq, &c, &scale};
    const void* fn;
    int threads = 64 * NW;
    if constexpr (D == 128 && NW == 8) {  // the eight-wave shape: always the ping-pong dQ
      fn = reinterpret_cast<const void*>(&attn_bwd_dq_pp_kernel<E, CAUSAL>);
      threads = 512;
    } else if constexpr (D == 128) {
      fn = a.dq_pp ? reinterpret_cast<const void*>(&attn_bwd_dq_pp_kernel<E, CAUSAL>)
                   : reinterpret_cast<const void*>(&attn_bwd_dq_kernel<E, D, CAUSAL, NW>);
      threads = a.dq_pp ? 512 : 64 * NW;
    } else {
      fn = reinterpret_cast<const void*>(&attn_bwd_dq_kernel<E, D, CAUSAL, NW>);
    }
    const hipError_t err = hipLaunchKernel(fn, dim3(BH * nq), dim3(threads), args, 0, a.stream);
    if (err != hipSuccess) return err;
  }
  if (nk > 0) {
    void* args[] = {&q, &k, &v, &lse, &d_o, &delta, &dk, &dv, &BH, &Nq, &Nk, &nk, &c, &scale};
    auto go = [&](const void* fn) {
      return hipLaunchKernel(fn, dim3(BH * nk), dim3(64 * NW), args, 0, a.stream);
    };
    if constexpr (D == 256) {
      const hipError_t err =
          go(reinterpret_cast<const void*>(&attn_bwd_kv_kernel<E, D, CAUSAL, NW, 1>));
      if (err != hipSuccess) return err;
      return go(reinterpret_cast<const void*>(&attn_bwd_kv_kernel<E, D, CAUSAL, NW, 2>));
    } else {
      return go(reinterpret_cast<const void*>(&attn_bwd_kv_kernel<E, D, CAUSAL, NW>));
    }
  }
  return hipSuccess;
}


}  // namespace
