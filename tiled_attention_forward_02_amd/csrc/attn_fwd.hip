// attn_fwd.hip - fused attention forward for gfx950 (CDNA4) and its C ABI.
//
// What it computes is the tiled, fused attention of "[GPU] Deep Learning for
// HPC", section "Flash Attention": the score matrix is cut into tiles that
// never leave the chip; softmax (null-ptr.tistory.com, category "development",
// softmax post: e^{z_i} / sum_j e^{z_j}, maximum subtracted against overflow)
// is carried across key tiles with a running maximum and a running sum; the
// per-row log-sum-exp is written next to the output, as in the Triton forward
// signature on that same page (Out, Lse, softmax_scale, IS_CAUSAL).
//
// Design for MI355X (gfx950). One workgroup of 4 waves owns 128 query rows of
// one (batch, head), each wave 32 of them, or at d = 128 256 rows, each wave
// two blocks of 32 that share every K and V fragment it reads from LDS. Two
// (d=128), three (d=96) or four (d=64) workgroups share a CU, so each SIMD
// holds waves of different workgroups whose softmax (VALU) and matrix (MFMA)
// phases interleave. On big grids (d = 96 and 128, d = 64 on long rows:
// 512-row workgroups; d = 256: 256 rows) a separate kernel (further down)
// runs eight waves whose two groups alternate the two kinds of work by
// barrier, a phase apart; d = 32 runs eight one-block waves there. Keys and
// values stream through LDS in tiles of 32 (d=128) or 64 (d=64) keys, double
// buffered one tile ahead with one barrier per tile: at d = 64, 96, 128 and
// 256 both, by buffer loads that write LDS directly (LDS DMA),
// each tile through a buffer resource based at its first row; the rest
// HBM -> registers -> LDS. Global loads are buffer loads: rows past N come
// back as zeros, with no branches. Both contractions run on
// v_mfma_f32_32x32x16_bf16 in transposed form:
//
//   S^T (keys x queries) = K (keys x d) * Q^T (d x queries)
//   O^T (d x queries)   += V^T (d x keys) * P^T (keys x queries)
//
// so one query sits in each lane (lane % 32) of both accumulators: the row
// statistics are per-lane scalars plus one swap between the two 32-lane
// halves, and the S^T accumulator rounded to bf16 is already the B operand of
// the P*V product, given a fixed permutation of the key order inside each
// 16-key slice. V stays row-major in LDS; transposing LDS reads
// (ds_read_b64_tr_b16) hand each lane the V^T column it needs, 4 keys at a
// time, in that permuted order.
//
// The running maximum is raised lazily. The first tile's row maximum is the
// first reference (O and the row sum are still zero then). After that, at
// d >= 64 the weights of a tile are computed against the current reference
// maximum straight away, and the reference moves (the tile's row maximum
// taken, O and the row sum rescaled, the weights redone) only when a lane's
// share of the tile's weights exceeds 2^12. At d = 32 the tile's row maximum
// comes first, and the reference moves only when it exceeds the reference by
// more than 2^8 (log2 units). Either way O / l and m + log2(l) stay exact in real
// arithmetic, because O and l always share one reference maximum. Masking
// (causal diagonal tiles and the tile holding key N-1) is the only
// per-element select, and only those tiles run it.
//
// The MFMA fragment layout these comments refer to is described in common.h.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <float.h>
#include <string.h>

#include <type_traits>

#include "common.h"
#include "mi_attn.h"

namespace {

using namespace mi_attn;

constexpr float kLazyMax = 8.0f;  // tolerated growth of the row max, log2 units
constexpr float kLazySum = 4096.f;  // largest per-lane tile sum kept on a stale max
// Softmax weights first, row maximum only when they grow too large, or row
// maximum first. Weights first saves the max reduction: measured faster at
// d = 64 to 256; at d = 32 slower (-0.9% to -3.4%), where the extra live
// scores cost more than the reduction. At d = 64 it takes the kernel from 4
// to 3 waves per SIMD and still wins (with the wave priority below, measured
// interleaved: +2.0% on B=4 H=16 N=1024, +3.1% on B=16 H=16 N=4096, +3.8% on
// the long causal shape, -0.7% on causal B=8 H=16 N=2048).
template <int D>
constexpr bool kSpeculativeWeights = D >= 64;
// Raise a wave's priority while it issues its two MFMA chains (and drop it
// for the softmax and the staging), so that when several waves of a SIMD
// have work the matrix pipe is fed first: +1.2-2.2% at d = 128 with one
// query block per wave (measured interleaved against the plain kernel); at
// d = 64 with weights first part of the gain above; at d = 32 not kept. With
// two query blocks per wave (d = 128, two waves per SIMD) it gains nothing
// (+0.1%, and -0.7% on the long causal shape), so it is left out there.
template <int D, int QB>
constexpr bool kMfmaPriority = D >= 64 && QB == 1;
// Stage K and V by buffer loads that write LDS directly (no registers, no
// LDS write instructions) instead of through registers. Timing copies that
// drop the global loads but keep the LDS writes ran 16% faster at d = 128:
// the loads into registers, not their latency, were the cost. Measured
// interleaved against the register path: K and V by DMA +2.2% at d = 128,
// +3.8% on the long causal workload, +7.5% at d = 96 (its kernel drops to
// 127 VGPRs, four waves per SIMD); at d = 64, with four waves per SIMD
// forced (kMinBlocks), +0.8% to +3.3% on four shapes (without the fourth
// wave -1.4% to +0.8%); at d = 32 DMA loses (-1%). At d = 256, with V's
// staging registers gone the kernel fits in 247 VGPRs, two waves per SIMD
// instead of one (404 registers with V through registers): +59% on
// B=16 H=16 N=4096 and +54% on the long causal shape (interleaved A/B,
// bit-identical outputs).
template <int D>
constexpr bool kKDma = D == 64 || D == 96 || D == 128 || D == 256;
template <int D>
constexpr bool kVDma = D == 64 || D == 96 || D == 128 || D == 256;
// DMA tiles are addressed through a resource based at the tile's first row
// rather than by adding the row offset to every lane's offset (two vector
// adds per DMA instruction, ten per tile and wave at d = 128). Measured
// interleaved: +1.4% at d = 128, +0.9% on the long causal d = 128 shape,
// +2.3% and +1.8% on two non-causal d = 64 shapes, +2.8% at d = 96, +1.8% at
// d = 256, and with the bit-select mask below +1.4% on causal d = 64.

// Workgroup shapes: QB 32-query blocks per wave, NW waves per workgroup (the
// 512-row shape at d = 64, 96 and 128, QB = 2 and NW = 8, and the 256-row
// shape at d = 256 run the ping-pong kernel).
// d = 32 and 256 have two, chosen at launch by the size of the grid: eight
// waves of one block (256 rows) on big grids, which halves the HBM -> LDS
// staging per FLOP, else four waves. At d = 256 (one per CU, two waves per
// SIMD) that gave +3.9% and +6.7% on B=16 H=16 N=4096 and the long causal
// shape, at d = 32 (two per CU) +3.5% and +2.3% (interleaved A/Bs); at d = 96
// (two per CU, four waves per SIMD) +2.7% and +3.4%, before the ping-pong
// kernel's 512 rows replaced it there (a further +2.9% to +8.5% on four
// shapes). At d = 256 the ping-pong kernel then ran those eight waves 1.9%
// and 2.7% faster than this kernel. At d = 64 eight waves gained +0.5% on big
// grids and lost 2.6-2.8% on the two small workloads, so d = 64 keeps four
// outside the ping-pong kernel's long rows. d = 128 has three:
// - QB = 2, NW = 8 (512 rows a workgroup, one per CU, two waves per SIMD),
//   in the ping-pong kernel: +8.9% on B=16 H=16 N=4096 and +9.5% on the long
//   causal shape over the same shape run by this kernel, whose two waves of a
//   SIMD did the same kind of work at the same time (interleaved A/B,
//   bit-identical outputs);
// - QB = 2, NW = 4 (256 rows, two per CU, two waves per SIMD);
// - QB = 1, NW = 4 (128 rows, three per CU, three waves per SIMD).
// With two blocks a wave, every K and V^T fragment it reads from LDS serves
// both, which halves the LDS read traffic per FLOP; the kernel then fits in
// 256 VGPRs, two waves per SIMD. Under the power cap that beat three
// one-block waves per SIMD by 3.0% and 6.1% on B=16 H=16 N=4096 on two boxes,
// and by 2.2% on the long causal shape. Eight waves a workgroup then halve
// the HBM -> LDS staging per FLOP again: a further +2.0% and +0.9% (all
// interleaved A/Bs, bit-identical outputs). Bigger workgroups mean fewer of
// them, so small grids keep the smaller shapes. In this kernel two blocks a
// wave lost to the fourth one-block wave per SIMD at d = 96 (-1.1%, -6%) and
// d = 64 (-12% on the two small workloads), so below the ping-pong kernel's
// shapes every other d runs QB = 1, NW = 4.
// Workgroups per CU the register allocation must allow.
template <int D, int QB, int NW>
constexpr int kMinBlocks =
    QB == 2 ? 8 / NW
    : NW == 8 ? (D == 256 ? 1 : 2)  // eight waves (d = 32 only): two a CU
              : (D == 64 ? 4 : D == 96 || D == 128 ? 3 : 2);
// The most query rows a workgroup has (the 32-bit offset check on Nq allows
// for one workgroup's rows past the end).
constexpr int kBlockMMax = 32 * 8 * 2;
// Keys per tile for head dimension D. At d=128 a 32-key tile keeps a
// two-block wave within 256 VGPRs (two waves per SIMD) and a workgroup at
// 38 KiB of LDS; at d=96 a one-block wave within 128 (four per SIMD); at
// d=64 a 64-key tile already fits four.
template <int D>
constexpr int kBlockN = 64;
template <>
constexpr int kBlockN<32> = 128;  // each thread still stages 2 keys of 8 columns
template <>
constexpr int kBlockN<96> = 32;
template <>
constexpr int kBlockN<128> = 32;
template <>
constexpr int kBlockN<256> = 32;

// Head dimension of the LDS tile layout: d = 96 tiles are laid out as d = 128
// ones (12 of 16 chunks per row staged and read), so the 256 threads still
// stage two rows of one 16-byte chunk each; no MFMA work is padded.
template <int D>
constexpr int kLayoutD = D == 96 ? 128 : D;

// Per head dimension D and tile width BN: the key tile and its LDS layout.
// At d = 64 the rows are unpadded and swizzled (kSwz; see the DMA below),
// which made its transposing reads conflict-free (0.333 conflict cycles per
// LDS-active cycle before, at a V pitch of 80) and needs two DMA source
// offsets a lane instead of six: +3.3% on B=4 H=16 N=1024 and +2.5% on
// causal B=8 H=16 N=2048 (interleaved A/B, bit-identical outputs).
template <int D>
constexpr bool kSwz = D == 64;
template <int D, int BN_, int NW = kWaves>
struct Tile {
  static constexpr int BN = BN_;
  static constexpr int NKB = BN / 32;            // 32-key MFMA blocks per tile
  // K row pitch in LDS (bf16): a 16 B pad, or none with the swizzled layout
  static constexpr int KS = kSwz<D> ? D : D + 8;
  static constexpr int K_ELEMS = BN * KS;        // one K tile
  // LDS span of a K tile: rounded up to 1024 bytes, so that DMA instructions
  // (1024 bytes each) that run past the tile write its padding, not V.
  static constexpr int K_SPAN = (K_ELEMS + 511) / 512 * 512;
  static constexpr int VS = kSwz<D> ? D : tr_pitch<D>();  // V row pitch in LDS
  static constexpr int V_ELEMS = BN * VS;        // one V tile, row-major
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  // Rows each thread stages through registers (d = 32 and the V tile at
  // d = 256, both with four waves; the other shapes stage by DMA).
  static constexpr int KPT = BN * CPR / (64 * NW) > 0 ? BN * CPR / (64 * NW) : 1;
  static constexpr int STAGE = K_SPAN + V_ELEMS;
  static constexpr int LDS_ELEMS = 2 * STAGE;
  static constexpr int LDS_BYTES = 2 * LDS_ELEMS;
  static_assert(NW != kWaves || KPT == 2 || KPT == 4, "staging layout");
};

template <typename E, int D, bool CAUSAL, int QB, int NW>
__global__ __launch_bounds__(64 * NW, (kMinBlocks<D, QB, NW>)) void attn_fwd_kernel(
    const E* __restrict__ Q, const E* __restrict__ K,
    const E* __restrict__ V, E* __restrict__ O,
    float* __restrict__ LSE, int BH, int Nq, int Nk, int nq, float c) {
  using T = Tile<kLayoutD<D>, kBlockN<D>, NW>;
  constexpr int BN = T::BN, KS = T::KS, CPR = T::CPR, KPT = T::KPT, NKB = T::NKB;
  // Chunks of a row that hold data (all but the layout's padding at d = 96).
  constexpr int CPR_DATA = D / 8;
  typedef typename Elem<E>::v8 v8;
  typedef typename Elem<E>::v4 v4;
  __shared__ __attribute__((aligned(1024))) E smem[T::LDS_ELEMS];

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave; readfirstlane lets the
  // compiler keep it (and what follows from it) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;

  constexpr int kBlockM = 32 * NW * QB;
  int bh, qt;
  map_block(blockIdx.x, BH, nq, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  const int qw = q0 + 32 * QB * wave;  // first query row of this wave
  // This lane's query row in block b is qw + 32 b + col.

  // Query rows live on [0, Nq), keys on [0, Nk); query i sits at key position
  // i + off (the two axes aligned at their ends; off = 0 when Nq == Nk).
  const int off = Nk - Nq;
  const size_t qhead = (size_t)bh * (size_t)Nq * D;
  const size_t khead = (size_t)bh * (size_t)Nk * D;
  const uint32_t q_bytes = (uint32_t)Nq * D * 2;
  const uint32_t k_bytes = (uint32_t)Nk * D * 2;
  const rsrc_t rq = make_rsrc(Q + qhead, q_bytes);
  const rsrc_t rk = make_rsrc(K + khead, k_bytes);
  const rsrc_t rv = make_rsrc(V + khead, k_bytes);

  // Q^T fragments (B operand): lane holds Q[qi][16s + 8h .. +7] of its row
  // qi in each block; zero past N.
  u32x4 qraw[QB][D / 16];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qraw[b][s] = load16(rq, (uint32_t)((qw + 32 * b + col) * D + 16 * s + 8 * half) * 2);
  // Fold the sign of the scale into Q (exact) so that c > 0 below: then a
  // masked score of -inf gets weight exp2(-inf) = 0 and the row max skips it.
  // scale == 0 makes every score 0, the same as Q == 0 with any scale.
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[b][s] ^= 0x80008000u;
  } else if (c == 0.f) {
    c = 1.f;
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[b][s] = u32x4{0, 0, 0, 0};
  }
  v8 qf[QB][D / 16];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[b][s] = __builtin_bit_cast(v8, qraw[b][s]);

  // Keys this workgroup / this wave can see (none for rows before -off).
  const int kv_end = CAUSAL ? min(Nk, q0 + kBlockM + off) : Nk;
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const int wave_kv_end = CAUSAL ? min(Nk, qw + 32 * QB + off) : Nk;

  char* const lds = reinterpret_cast<char*>(smem);

  // Staging by DMA (DmaTile): K and V tiles straight from HBM into LDS, no
  // registers; the K tile's LDS span is rounded up to 1024 bytes for it.
  typedef DmaTile<D, BN, KS, NW> KDma;
  typedef DmaTile<D, BN, T::VS, NW> VDma;
  static_assert(kSwz<D> || KDma::SPAN == T::K_SPAN * 2, "K DMA span is the K tile's LDS span");
  static_assert(kSwz<D> || !kVDma<D> || VDma::SPAN == T::V_ELEMS * 2,
                "V DMA covers the V tile exactly");
  lds_char* const lds3 = to_lds(smem);
  const KDma kdma(wave, lane);
  const VDma vdma(wave, lane);
  // Swizzled layout (d = 64): rows of 128 bytes without padding; K keeps
  // 16-byte chunk c of row r at c ^ ((r >> 1) & 7), V 64-byte group g at
  // g ^ ((r >> 1) & 1). A tile part is 8 DMA instructions (8 rows each);
  // wave w issues u = w and w + 4 of K and of V, each half tile (32 rows)
  // through a resource based at its first row (rows past Nk read as zeros).
  // Within a wave the swizzles depend on the lane only, so one source offset
  // serves both of its instructions of a part.
  uint32_t sw_k = 0, sw_v = 0;
  if constexpr (kSwz<D>) {
    const int r = 8 * wave + (lane >> 3), pc = lane & 7;
    sw_k = (uint32_t)(r * D * 2 + 16 * (pc ^ ((r >> 1) & 7)));
    sw_v = (uint32_t)(r * D * 2 + 16 * (4 * ((pc >> 2) ^ ((r >> 1) & 1)) + (pc & 3)));
  }
  auto dma = [&](auto stage_c, int k0) {
    constexpr uint32_t base = decltype(stage_c)::value * T::STAGE * 2;
    if constexpr (kSwz<D>) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r0 = k0 + 32 * i;
        const uint32_t n = r0 < Nk ? (uint32_t)(Nk - r0) * D * 2 : 0u;
        const uint32_t at = base + 1024 * (wave + 4 * i);
        load16_lds(make_rsrc(K + khead + (size_t)r0 * D, n), lds3 + at, sw_k);
        load16_lds(make_rsrc(V + khead + (size_t)r0 * D, n), lds3 + at + T::K_SPAN * 2, sw_v);
      }
      return;
    }
    // The tile's first row goes into the resource's base and its records
    // count from there, so placing the tile is scalar work; rows past Nk
    // still come back as zeros.
    const uint32_t skip = (uint32_t)k0 * D * 2;
    if constexpr (kKDma<D>)
      kdma.issue(make_rsrc(K + khead + (size_t)k0 * D, k_bytes - skip), lds3 + base, wave);
    if constexpr (kVDma<D>)
      vdma.issue(make_rsrc(V + khead + (size_t)k0 * D, k_bytes - skip),
                 lds3 + base + T::K_SPAN * 2, wave);
  };

  // Staging through registers: thread owns rows kr .. kr+KPT-1 and 16-byte
  // chunk dc of both K (register form) and V, the chunk fastest across lanes
  // (a row per CPR lanes: coalesced loads, contiguous 16-byte LDS writes).
  // Both tiles stay row-major in LDS; the V^T operand comes from
  // transposing reads.
  const int kr = KPT * (tid / CPR);
  const int dc = tid % CPR;
  const uint32_t goff = (uint32_t)(kr * D + 8 * dc) * 2;
  u32x4 kst[KPT], vst[KPT];

  // Chunks past the data (d = 96) are neither loaded nor read back.
  const bool data = CPR_DATA == CPR || dc < CPR_DATA;
  const bool k_data = !kKDma<D> && data;
  const bool v_data = !kVDma<D> && data;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t row = (uint32_t)((k0 + i) * D * 2);
      if (k_data) kst[i] = load16(rk, goff + row);
      if (v_data) vst[i] = load16(rv, goff + row);
    }
  };
  // Per-lane LDS byte offsets that do not change with the tile.
  const uint32_t k_wr = (uint32_t)(kr * KS + 8 * dc) * 2;
  const uint32_t v_wr = (uint32_t)(T::K_SPAN + kr * T::VS + 8 * dc) * 2;
  const uint32_t k_rd = kSwz<D> ? (uint32_t)(col * D * 2 + 16 * (half ^ ((col >> 1) & 7)))
                                : (uint32_t)(col * KS + 8 * half) * 2;
  // V^T operands come from transposing reads of the row-major V tile, two
  // per 16-key slice (tr_operand): the keys in the order of the P^T slots.
  uint32_t v_rd = (uint32_t)T::K_SPAN * 2 + tr_lane_off<T::VS>(lane);
  if constexpr (kSwz<D>) {
    const int g = lane >> 4, s = lane & 15, rl = 4 * (g >> 1) + (s >> 2);
    v_rd = (uint32_t)T::K_SPAN * 2 +
           (uint32_t)(rl * D * 2 + 64 * ((rl >> 1) & 1) + 32 * (g & 1) + 8 * (s & 3));
  }

  auto lds_store = [&](auto stage_c) {
    constexpr uint32_t base = decltype(stage_c)::value * T::STAGE * 2;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (k_data) *reinterpret_cast<u32x4*>(lds + base + k_wr + i * KS * 2) = kst[i];
      if (v_data) *reinterpret_cast<u32x4*>(lds + base + v_wr + i * T::VS * 2) = vst[i];
    }
  };

  f32x16 oacc[QB][D / 32];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[b][db] = f32x16{};
  // Reference maximum of O and l (log2 units), per block. It starts at
  // -FLT_MAX, not -inf, so that a row with no visible key keeps l = 0
  // without NaN.
  float m_run[QB], l_run[QB];  // l_run: this lane's share of the row sum
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m_run[b] = -FLT_MAX;
    l_run[b] = 0.f;
  }

  // One tile: S^T, mask, running max, P, O^T += V^T P^T; then stage the next.
  // `first_c`: the first tile (t = 0), which every wave that sees a key
  // computes.
  auto step = [&](int t, auto stage_c, auto first_c) {
    constexpr int stage = decltype(stage_c)::value;
    constexpr bool first = decltype(first_c)::value;
    constexpr uint32_t base = stage * T::STAGE * 2;
    const int k0 = t * BN;
    const bool has_next = t + 1 < nt;
    if (has_next) {
      dma(std::integral_constant<int, stage ^ 1>{}, k0 + BN);
      gload(k0 + BN);
    }

    if (k0 < wave_kv_end && qw < Nq) {
      if constexpr ((kMfmaPriority<D, QB>)) __builtin_amdgcn_s_setprio(1);
      // S^T = K * Q^T: NKB blocks of 32 keys, one MFMA chain each per query
      // block; each K fragment read from LDS serves every query block.
      f32x16 sacc[QB][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int b = 0; b < QB; ++b) sacc[b][kb] = f32x16{};
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const v8 a = kSwz<D>
              ? *reinterpret_cast<const v8*>(lds + base + 32 * kb * D * 2 + (k_rd ^ (32u * j)))
              : *reinterpret_cast<const v8*>(lds + base + k_rd + (32 * kb * KS + 16 * j) * 2);
#pragma unroll
          for (int b = 0; b < QB; ++b) sacc[b][kb] = Elem<E>::mfma(a, qf[b][j], sacc[b][kb]);
        }
      }

      if constexpr ((kMfmaPriority<D, QB>)) __builtin_amdgcn_s_setprio(0);
      // Keys past the end and (causal) keys after the query get -inf.
      // Register i of block kb holds key k0 + 4 half + o_i. With 32 or more
      // scores a lane (d = 32 and 64, and d = 128 with two query blocks) a
      // bit select on the sign of lim - o_i, lim being the last key the
      // lane's query sees less k0 + 4 half: compares would hold a lane mask
      // (two SGPRs) per score until its select, and the SGPRs spill (at
      // d = 64 the causal kernel spilled 18 SGPRs and 3 VGPRs; without them
      // it ran 3.3% faster on causal B=8 H=16 N=2048, measured interleaved;
      // at d = 128 it spilled 40). With 16 scores a lane a compare and
      // select per score (the bit select costs VGPRs there: at d = 96 it
      // would cost the fourth wave per SIMD).
      if ((k0 + BN > Nk) || (CAUSAL && k0 + BN - 1 > qw + off)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const int qi = qw + 32 * b + col;
          if constexpr (NKB * 16 * QB >= 32) {
            const int lim = (CAUSAL ? min(Nk - 1, qi + off) : Nk - 1) - k0 - 4 * half;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int o = 32 * kb + 8 * (i >> 2) + (i & 3);
                sacc[b][kb][i] = neg_inf_where((lim - o) >> 31, sacc[b][kb][i]);
              }
          } else {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
                if (key >= Nk || (CAUSAL && key > qi + off)) sacc[b][kb][i] = -INFINITY;
              }
          }
        }
      }

      // P = 2^(s*c - m_run), rounded to bf16, and its row sum (fp32).
      v8 pb[QB][NKB][2];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        float tsum = 0.f;
        auto weights = [&]() __attribute__((always_inline)) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(sacc[b][kb][i], c, -m_run[b]));
              // The sum starts at the first weight: 0 + p is not folded when
              // signed zeros are honoured, and would cost an add per tile
              // (+0.2% to +0.8% measured interleaved without it).
              if (kb == 0 && i == 0)
                tsum = p;
              else
                tsum += p;
              pb[b][kb][i >> 3][i & 7] = (E)p;
            }
        };
        // Row maximum of the tile in log2 units, both lane halves combined.
        auto tile_max = [&]() __attribute__((always_inline)) {
          float mx = fmaxf(sacc[b][0][0], sacc[b][0][1]);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = kb ? 0 : 2; i < 16; i += 2)
              mx = fmaxf(mx, fmaxf(sacc[b][kb][i], sacc[b][kb][i + 1]));
          return swap_halves_max(mx) * c;
        };
        // Move O and l to a new reference maximum.
        auto rebase = [&](float m_new) __attribute__((always_inline)) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
          l_run[b] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[b][db] *= alpha;
          m_run[b] = m_new;
        };
        if constexpr (first) {
          // The tile's row maximum becomes the reference. O and l are still
          // zero, so there is nothing to rescale (a rebase would multiply
          // them by 0, or by 1 in a row that sees none of the tile's keys).
          m_run[b] = fmaxf(m_run[b], tile_max());
          weights();
        } else if constexpr (kSpeculativeWeights<D>) {
          // Weights against the current reference, without the tile's own
          // maximum. The reference moves only when this lane's share of the
          // tile's weights exceeds kLazySum (every weight then stayed below
          // it): the tile's true row maximum becomes the reference and the
          // weights are redone.
          weights();
          if (__any(tsum > kLazySum)) {
            rebase(fmaxf(m_run[b], tile_max()));
            weights();
          }
        } else {
          // Move the reference only when the tile's row maximum exceeds it by
          // more than kLazyMax.
          const float m_tile = tile_max();
          if (__any(m_tile > m_run[b] + kLazyMax)) rebase(fmaxf(m_run[b], m_tile));
          weights();
        }
        l_run[b] += tsum;
      }

      if constexpr ((kMfmaPriority<D, QB>)) __builtin_amdgcn_s_setprio(1);
      // O^T += V^T * P^T, 16 keys per MFMA; each V^T fragment serves every
      // query block.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            v8 a;
            if constexpr (kSwz<D>) {
              const char* p = lds + base + (v_rd ^ (64u * db)) + (32 * kb + 16 * sg) * D * 2;
              const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * D * 2);
              a = __builtin_bit_cast(v8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            } else {
              a = tr_operand<v8, T::VS>(lds + base, v_rd, 32 * kb + 16 * sg, 32 * db);
            }
#pragma unroll
            for (int b = 0; b < QB; ++b) oacc[b][db] = Elem<E>::mfma(a, pb[b][kb][sg], oacc[b][db]);
          }
        }
    }

    if constexpr ((kMfmaPriority<D, QB>)) __builtin_amdgcn_s_setprio(0);
    if (has_next) lds_store(std::integral_constant<int, stage ^ 1>{});
    // DMA form: the next tile's K lands in LDS with no instruction of this
    // wave writing it; wait for the loads before the barrier.
    if constexpr (kKDma<D> || kVDma<D>) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  dma(std::integral_constant<int, 0>{}, 0);
  gload(0);
  lds_store(std::integral_constant<int, 0>{});
  if constexpr (kKDma<D> || kVDma<D>) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nt > 0) step(0, std::integral_constant<int, 0>{}, std::true_type{});
  for (int t = 1; t < nt; t += 2) {
    step(t, std::integral_constant<int, 1>{}, std::false_type{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 0>{}, std::false_type{});
  }

  // Epilogue: O = acc / l (bf16), lse = (m + log2 l) * ln 2. Rows past N are
  // dropped by the buffer range check.
  const rsrc_t ro = make_rsrc(O + qhead, q_bytes);
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int qi = qw + 32 * b + col;
    const float total = swap_halves_add(l_run[b]);
    // A row that saw no key (l = 0) gets O = 0 and lse = -inf.
    const float inv = total > 0.f ? 1.0f / total : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (E)(oacc[b][db][4 * r + e] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), ro,
                                              (int)((qi * D + 32 * db + 8 * r + 4 * half) * 2),
                                              0, 0);
      }
    }
    if (half == 0) {
      const float lse = total > 0.f ? (m_run[b] + log2f(total)) * kLn2 : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qi * 4, 0, 0);
    }
  }
}

// ----------------------------- ping-pong kernel (d = 64, 96, 128, 256, big grids) --
// 512 query rows a workgroup of 8 waves, two 32-query blocks a wave (256 rows,
// one block a wave, at d = 256); waves w and w + 4 share a SIMD. Each wave
// alternates an MFMA phase M(t) (O^T += V^T P^T of tile t-1, then
// S^T = K Q^T of tile t) and a softmax phase X(t) (mask, weights, row sums of
// tile t), with a workgroup barrier after each; waves 4-7 run one phase
// behind waves 0-3, so on every SIMD one wave's matrix work runs beside the
// other's softmax instead of both waves doing the same kind of work at once.
// The MFMA phase must then keep the matrix pipe fed on its own: its LDS
// operands are read three MFMAs ahead (the first fragments of M(t+1) at the
// end of X(t), the first K fragments during the last P*V MFMAs), and the tile
// DMA is issued between MFMAs without a branch. At d = 256 a wave's one S
// chain of 16 dependent MFMAs would stall the pipe, so its steps alternate
// with the P*V MFMAs.
//
// Tiles of 8 KiB of K and 8 of V (32 keys at d = 128, 64 at d = 64; 16 KiB
// each of 32 keys at d = 256; at d = 96 32 keys laid out as at d = 128, whose
// chunks 12-15 of each row the DMA fills with zeros and no read touches),
// rows without padding, in a ring of three LDS stages (K at +0, V after it).
// K keeps 16-byte chunk c of row r at chunk c ^ (r & 15) (d >= 96) or
// c ^ ((r >> 1) & 7) (d = 64), so the 16 rows one pass of a 16-byte read
// covers hit all 64 banks (rows 256 or 512 bytes apart would otherwise all
// start on bank 0); V keeps 64-byte group g of row r at g ^ (r & 3)
// (d >= 96) or g ^ ((r >> 1) & 1) (d = 64), so the 4 rows one pass of a
// transposing read covers do. Both swizzles depend on the lane only through
// lane / 16, the wave and (K at d = 256) whether the DMA instruction is the
// odd one of its pair, so each wave's DMA instructions of a tile part need
// at most two per-lane source offsets.
template <typename E, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_fwd_pp_kernel(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V, E* __restrict__ O,
    float* __restrict__ LSE, int BH, int Nq, int Nk, int nq, float c) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 256,
                "the ping-pong kernel: d = 64, 96, 128, 256");
  constexpr int QB = D == 256 ? 1 : 2, NW = 8, NST = 3;
  constexpr int BN = D == 64 ? 64 : 32;       // keys per tile: 8 KiB of K, 8 of V (16 at d = 256)
  constexpr int NKB = BN / 32;                // 32-key blocks per tile
  // The MFMA phase runs at raised wave priority, so that its MFMAs go first
  // when the softmax wave of the SIMD also has work; not at d = 64, whose
  // softmax phase is the longer one (without it +0.7% to +1.6% on three
  // d = 64 shapes, two boxes; with it at d = 128, 96 and 256 +0.6% to +3.8%).
  constexpr bool kPhasePrio = D != 64;
  constexpr int NDB = D / 32;                 // 32-column blocks of O
  constexpr int DL = D == 96 ? 128 : D;       // row width in LDS (d = 96: chunks 12-15 zero)
  constexpr uint32_t ROWB = DL * 2;           // bytes per row in LDS
  constexpr uint32_t GROWB = D * 2;           // bytes per row in HBM
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;            // rows per DMA instruction
  constexpr int HALF = 4 * RPI;               // rows per 4-wave DMA round
  constexpr uint32_t TB = BN * ROWB;          // bytes per K or V tile
  constexpr uint32_t SB = 2 * TB;             // bytes per stage
  constexpr int NI = TB / 4096;               // DMA instructions a wave per tile part
  static_assert(TB % 8192 == 0 && NI * HALF == BN, "whole DMA rounds per tile part");
  constexpr int NPV = 2 * NDB * NKB;          // P*V MFMAs (operand fragments) per tile
  constexpr int NSG = D / 16 * NKB;           // S MFMAs (operand fragments) per tile
  // Swizzles: K chunk c of row r sits at c ^ kswz(r), V 64-byte group g at
  // g ^ vswz(r); within one wave's DMA instructions both depend on r only
  // through lane / 16 and (K at d = 256) whether the instruction is even.
  auto kswz = [](int r) { return DL >= 128 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return DL >= 128 ? (r & 3) : ((r >> 1) & 1); };
  typedef typename Elem<E>::v8 v8;
  typedef typename Elem<E>::v4 v4;
  __shared__ __attribute__((aligned(1024))) char smem[NST * SB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const bool late = wave >= 4;
  const int dwave = wave & 3;

  constexpr int kBlockM = 32 * NW * QB;
  int bh, qt;
  map_block(blockIdx.x, BH, nq, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  const int qw = q0 + 32 * QB * wave;
  const int off = Nk - Nq;
  const size_t qhead = (size_t)bh * (size_t)Nq * D;
  const size_t khead = (size_t)bh * (size_t)Nk * D;
  const uint32_t q_bytes = (uint32_t)Nq * D * 2;
  const rsrc_t rq = make_rsrc(Q + qhead, q_bytes);

  u32x4 qraw[QB][D / 16];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qraw[b][s] = load16(rq, (uint32_t)((qw + 32 * b + col) * D + 16 * s + 8 * half) * 2);
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[b][s] ^= 0x80008000u;
  } else if (c == 0.f) {
    c = 1.f;
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qraw[b][s] = u32x4{0, 0, 0, 0};
  }
  v8 qf[QB][D / 16];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[b][s] = __builtin_bit_cast(v8, qraw[b][s]);

  const int kv_end = CAUSAL ? min(Nk, q0 + kBlockM + off) : Nk;
  const int nt = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // Tiles t < wave_nt hold a key this wave's rows see.
  const int wave_kv_end = qw < Nq ? (CAUSAL ? min(Nk, qw + 32 * QB + off) : Nk) : 0;
  const int wave_nt = wave_kv_end > 0 ? (wave_kv_end + BN - 1) / BN : 0;

  const char* const lds = smem;
  lds_char* const lds3 = to_lds(smem);

  // DMA source offsets of this lane (row RPI w' + lane / CPR of a DMA
  // round's HALF rows, the logical chunk its physical slot lane % CPR holds)
  // for even and odd instructions: K for the late waves, V for the early
  // ones. The two differ only for K at d = 256. At d = 96 a slot whose
  // logical chunk lies past the row's 12 gets an offset past any buffer:
  // zeros, no fetch.
  uint32_t dsrc[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int rl = RPI * dwave + lane / CPR, pc = lane % CPR, r = rl + HALF * e;
    const int ck = pc ^ kswz(r);
    const int cv = 4 * ((pc >> 2) ^ vswz(r)) + (pc & 3);
    const int lc = late ? ck : cv;
    dsrc[e] = lc < D / 8 ? (uint32_t)(rl * (int)GROWB + 16 * lc) : 0x80000000u;
  }
  // This wave's NI DMA instructions of the K (late waves) or V (early
  // waves) part of the tile from key k0, into the stage at byte `base`. Each
  // round of HALF rows goes through a resource based at its first row whose
  // record count ends at the head's last key (zero if it lies past it), so
  // rows past Nk come back as zeros. At d >= 128, where the MFMA phase is the
  // longer one, the resources are made one phase ahead (dma_prep, in the
  // softmax phase, whose VALU stream leaves issue slots free), so that the
  // MFMA phase only sets M0 and issues the loads: +4.8% at d = 256, +0.7% at
  // d = 128 (B=16 H=16 N=4096, interleaved). At d = 64 and 96 the softmax
  // phase is the longer one, and making them there lost 1.1% and 2.9%, so
  // the MFMA phase makes them right before the loads.
  constexpr bool kPrepAhead = D >= 128;
  rsrc_t dres[NI];
  auto dma_prep = [&](int k0) __attribute__((always_inline)) {
    const E* src = late ? K : V;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r0 = k0 + HALF * i;
      const uint32_t n = r0 < Nk ? (uint32_t)(Nk - r0) * GROWB : 0u;
      dres[i] = make_rsrc(src + khead + (size_t)r0 * D, n);
    }
  };
  auto dma_issue_one = [&](uint32_t base, int i) __attribute__((always_inline)) {
    const uint32_t part = late ? 0u : TB;
    load16_lds(dres[i], lds3 + base + part + 1024 * (dwave + 4 * i), dsrc[i & 1]);
  };
  auto dma_issue = [&](uint32_t base) __attribute__((always_inline)) {
    const uint32_t part = late ? 0u : TB;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      load16_lds(dres[i], lds3 + base + part + 1024 * (dwave + 4 * i), dsrc[i & 1]);
  };
  auto dma = [&](uint32_t base, int k0) __attribute__((always_inline)) {
    const E* src = late ? K : V;
    const uint32_t part = late ? 0u : TB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r0 = k0 + HALF * i;
      const uint32_t n = r0 < Nk ? (uint32_t)(Nk - r0) * GROWB : 0u;
      load16_lds(make_rsrc(src + khead + (size_t)r0 * D, n),
                 lds3 + base + part + 1024 * (dwave + 4 * i), dsrc[i & 1]);
    }
  };
  // Read bases: K fragment j of lane (col, half) is logical chunk 2 j + half
  // of row col, at kb ^ 32 j; V^T fragment (rows row0 .., columns 32 db ..)
  // at (vb ^ 64 db) + row0 * 256 (+ 8 rows for its second read).
  const uint32_t kb = (uint32_t)(col * (int)ROWB + 16 * (half ^ kswz(col)));
  uint32_t vb;
  {
    const int g = lane >> 4, s = lane & 15, rl = 4 * (g >> 1) + (s >> 2);
    vb = (uint32_t)(rl * (int)ROWB + 64 * vswz(rl) + 32 * (g & 1) + 8 * (s & 3)) + TB;
  }
  // The XORs are redone at each use (one VALU op each) rather than hoisted
  // out of the loop into eight more live registers: `kbase` and `vbase` pass
  // the bases through an empty asm once per phase, which the compiler cannot
  // see through.
  uint32_t kbl = kb, vbl = vb;
  auto refresh = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(kbl), "+v"(vbl));
  };
  // K fragment j: key block j / (D / 16), columns 16 (j % (D / 16)) ..;
  // V^T fragment i: key block i / (2 NDB), 16-key slice (i / NDB) % 2,
  // output columns 32 (i % NDB) ..
  auto kfrag = [&](uint32_t base, int j) __attribute__((always_inline)) {
    const int kbk = j / (D / 16), jj = j % (D / 16);
    return *reinterpret_cast<const v8*>(lds + base + kbk * 32 * ROWB + (kbl ^ (32u * jj)));
  };
  auto vfrag = [&](uint32_t base, int i) __attribute__((always_inline)) {
    const int kbk = i / (2 * NDB), sg = (i / NDB) % 2, db = i % NDB;
    const char* p = lds + base + (vbl ^ (64u * db)) + (32 * kbk + 16 * sg) * ROWB;
    const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * ROWB);
    return __builtin_bit_cast(v8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };

  f32x16 oacc[QB][NDB];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[b][db] = f32x16{};
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m_run[b] = -FLT_MAX;
    l_run[b] = 0.f;
  }
  // Weights of the last tile softmaxed (bf16), consumed by the next M phase,
  // and the first two V^T fragments of that tile, read at the end of the
  // softmax phase.
  v8 pb[QB][NKB][2];
  v8 vpre[D == 256 ? 4 : 3];

  // Mask, weights and row sums of tile t (its scores in sacc) into pb. The
  // two query blocks' weights are computed interleaved (the wave runs this
  // phase alone on its SIMD's VALU, so it needs the independent work); each
  // block's sum keeps its own order.
  auto softmax = [&](f32x16 (&sacc)[QB][NKB], int t, auto first_c)
      __attribute__((always_inline)) {
    constexpr bool first = decltype(first_c)::value;
    const int k0 = t * BN;
    if ((k0 + BN > Nk) || (CAUSAL && k0 + BN - 1 > qw + off)) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int qi = qw + 32 * b + col;
        const int lim = (CAUSAL ? min(Nk - 1, qi + off) : Nk - 1) - k0 - 4 * half;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int o = 32 * kb + 8 * (i >> 2) + (i & 3);
            sacc[b][kb][i] = neg_inf_where((lim - o) >> 31, sacc[b][kb][i]);
          }
      }
    }
    // Each block's row sum runs in four chains (weights i = 0, 1, 2, 3 mod 4),
    // added at the end, rather than one serial chain. At d = 64 and 96 one
    // test also covers both blocks' rebase, so that the compiler interleaves
    // the two blocks' weights instead of finishing one block before the
    // other's branch; at d = 128 that keeps too many values live across the
    // branch and spills, so each block keeps its own test there. Measured
    // interleaved: +0.7% at d = 64 (B=16 H=16 N=4096 and the long causal
    // shape), +0.3% and +0.4% on the two d = 128 workloads; the joint test
    // added +0.4% to +0.7% on four d = 96 shapes. This phase runs
    // on one wave of the SIMD, and one wave issues at most one VALU
    // instruction every ~9 cycles whatever the dependences (measured), so
    // its length is set by its instruction count.
    constexpr bool kJointRebase = D == 64 || D == 96;
    float tsum[QB], part[QB][4];
    auto weight = [&](int b, int kb, int i) __attribute__((always_inline)) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[b][kb][i], c, -m_run[b]));
      if (kb == 0 && i < 4)
        part[b][i] = p;
      else
        part[b][i & 3] += p;
      pb[b][kb][i >> 3][i & 7] = (E)p;
    };
    auto weights = [&](int b) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) weight(b, kb, i);
      tsum[b] = (part[b][0] + part[b][1]) + (part[b][2] + part[b][3]);
    };
    // The reference raised to the tile's row maximum (log2 units).
    auto raised = [&](int b) __attribute__((always_inline)) {
      float mx = fmaxf(sacc[b][0][0], sacc[b][0][1]);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = kb ? 0 : 2; i < 16; i += 2)
          mx = fmaxf(mx, fmaxf(sacc[b][kb][i], sacc[b][kb][i + 1]));
      return fmaxf(m_run[b], swap_halves_max(mx) * c);
    };
    auto rebase = [&](int b) __attribute__((always_inline)) {
      const float m_new = raised(b);
      const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
      l_run[b] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[b][db] *= alpha;
      m_run[b] = m_new;
      weights(b);
    };
    // The first tile's row maximum is the first reference; O and l are
    // still zero, so nothing is rescaled.
    if constexpr (first) {
#pragma unroll
      for (int b = 0; b < QB; ++b) m_run[b] = raised(b);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int b = 0; b < QB; ++b) weight(b, kb, i);
#pragma unroll
    for (int b = 0; b < QB; ++b) tsum[b] = (part[b][0] + part[b][1]) + (part[b][2] + part[b][3]);
    if constexpr (!first && kJointRebase) {
      float worst = tsum[0];
#pragma unroll
      for (int b = 1; b < QB; ++b) worst = fmaxf(worst, tsum[b]);
      // A block that did not need it is rebased too: exact, and rare.
      if (__any(worst > kLazySum)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) rebase(b);
      }
    } else if constexpr (!first) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
        if (__any(tsum[b] > kLazySum)) rebase(b);
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) l_run[b] += tsum[b];
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // O^T += V^T P^T of the V tile of the stage at `base`, fragments 0 and 1
  // already in vpre; fragment i + 2 is read while pair i runs.
  auto pv = [&](uint32_t base, auto tail) __attribute__((always_inline)) {
    v8 f[4] = {vpre[0], vpre[1], vpre[2], v8{}};
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + 3 < NPV) f[(i + 3) % 4] = vfrag(base, i + 3);
      const v8 a = f[i % 4];
      const int kbk = i / (2 * NDB), sg = (i / NDB) % 2, db = i % NDB;
#pragma unroll
      for (int b = 0; b < QB; ++b) oacc[b][db] = Elem<E>::mfma(a, pb[b][kbk][sg], oacc[b][db]);
      if (i == NPV - 3) tail();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // S^T = K Q^T of the K tile of the stage at `base`, fragments 0-2 in g
  // already; fragment j + 3 is read while pair j runs. `after0` runs after
  // the first pair.
  auto sgemm = [&](f32x16 (&sacc)[QB][NKB], uint32_t base, v8 (&g)[4], auto after0)
      __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NSG; ++j) {
      if (j + 3 < NSG) g[(j + 3) % 4] = kfrag(base, j + 3);
      const v8 a = g[j % 4];
      const int kbk = j / (D / 16), jj = j % (D / 16);
#pragma unroll
      for (int b = 0; b < QB; ++b)
        sacc[b][kbk] = jj == 0 ? Elem<E>::mfma(a, qf[b][jj], f32x16{})
                               : Elem<E>::mfma(a, qf[b][jj], sacc[b][kbk]);
      if (j == 0) {
        __builtin_amdgcn_sched_barrier(0);
        after0();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One tile t, stage st = t % 3 (phases 2t and 2t+1 for the early waves,
  // 2t+1 and 2t+2 for the late ones):
  //  M(t): O += P*V of tile t-1, then S of tile t. Between the two (after
  //        the transposing reads, which would otherwise wait for it) the
  //        early waves issue V of tile t+1 (its stage last read in the phase
  //        before), the late waves K of tile t+2 (into the stage of tile
  //        t-1, whose K part was last read two phases before).
  //  X(t): softmax of tile t into pb; read the first V^T fragments of tile t
  //        for the next M phase; wait for this wave's DMA, one phase or more
  //        before the first read of what it loaded.
  auto body = [&](int t, auto st_c, auto first_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    constexpr bool first = decltype(first_c)::value;
    constexpr uint32_t bcur = st * SB, bprev = ((st + 2) % NST) * SB;
    constexpr uint32_t bnext = ((st + 1) % NST) * SB;
    const bool do_s = t < wave_nt;
    refresh();
    if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(1);
    // The first three K fragments of tile t are read while the last P*V
    // pairs run (always: the stage holds tile t either way).
    v8 g[4];
    auto kread = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 3; ++j) g[j] = kfrag(bcur, j);
    };
    // The early waves load V of tile t+1 into the next stage, the late ones K
    // of tile t+2 into the previous one; issued without a branch (a tile past
    // the last one is loaded as zeros into a stage nobody reads again), after
    // the first S pair so that the matrix pipe has work meanwhile.
    auto issue_dma = [&]() __attribute__((always_inline)) {
      if constexpr (kPrepAhead)
        dma_issue(late ? bprev : bnext);
      else
        dma(late ? bprev : bnext, (t + (late ? 2 : 1)) * BN);
    };
    f32x16 sacc[QB][NKB];
    if constexpr (D == 256 && !first) {
      // One query block: the P*V MFMAs of tile t-1 and the S MFMAs of tile t
      // alternate, so that the chain of 16 dependent S MFMAs has an
      // independent MFMA between each two of its steps. Each MFMA needs an
      // operand of its own, read four MFMAs ahead; operands 0-3 (V^T 0, K 0,
      // V^T 1, K 1) were read at the end of the softmax phase before. The four
      // DMA instructions go one after each of the first four S steps (a wave
      // has few issue slots between two MFMAs). Against three operands ahead
      // and the DMA in one group: +0.3% to +1.2% on three d = 256 shapes, two
      // boxes (interleaved). A wave past its rows computes S anyway (the MFMA
      // stream has no branch) and drops it.
      v8 f[5] = {vpre[0], vpre[1], vpre[2], vpre[3], v8{}};
#pragma unroll
      for (int m = 0; m < 2 * NPV; ++m) {
        const int u = m + 4;
        if (u < 2 * NPV) f[u % 5] = (u & 1) ? kfrag(bcur, u / 2) : vfrag(bprev, u / 2);
        const v8 a = f[m % 5];
        if (m & 1) {
          const int j = m / 2;
          sacc[0][0] = j == 0 ? Elem<E>::mfma(a, qf[0][0], f32x16{})
                              : Elem<E>::mfma(a, qf[0][j], sacc[0][0]);
        } else {
          const int i = m / 2, sg = (i / NDB) % 2, db = i % NDB;
          oacc[0][db] = Elem<E>::mfma(a, pb[0][0][sg], oacc[0][db]);
        }
        if ((m & 1) && m / 2 < NI) {
          __builtin_amdgcn_sched_barrier(0);
          dma_issue_one(late ? bprev : bnext, m / 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // P*V of tile t-1 runs for every wave: one that skipped that tile holds
      // zero weights and adds exact zeros (its V rows are real data, or zeros
      // past the end). The first tile has no predecessor.
      if constexpr (first) {
        kread();
      } else {
        pv(bprev, kread);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_s) {
        sgemm(sacc, bcur, g, issue_dma);
      } else {
        issue_dma();
      }
    }
    if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(0);
    barrier();
    if constexpr (kPrepAhead) dma_prep((t + 1 + (late ? 2 : 1)) * BN);  // for M(t+1)
    if (do_s) {
      softmax(sacc, t, first_c);
    } else {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) pb[b][kb][0] = pb[b][kb][1] = v8{};
    }
    __builtin_amdgcn_sched_barrier(0);
    refresh();
    if constexpr (D == 256) {
      // K of tile t+1 was loaded in M(t-1) and waited for by the end of the
      // late waves' X(t-1).
      vpre[0] = vfrag(bcur, 0);
      vpre[1] = kfrag(bnext, 0);
      vpre[2] = vfrag(bcur, 1);
      vpre[3] = kfrag(bnext, 1);
    } else {
#pragma unroll
      for (int i = 0; i < 3; ++i) vpre[i] = vfrag(bcur, i);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA
    barrier();
  };

  // Prologue: V of tile 0 by the early waves, K of tiles 0 and 1 by the
  // late ones (in M(0) the early waves load V of tile 1, the late ones K of
  // tile 2); the late waves then wait one extra barrier, which puts them one
  // phase behind.
  if (nt > 0) dma(0, 0);
  if (late && nt > 1) dma(SB, BN);
  if constexpr (kPrepAhead) dma_prep((late ? 2 : 1) * BN);  // for M(0)
  __builtin_amdgcn_s_waitcnt(0);
  barrier();
  if (late) barrier();
  using no = std::false_type;
  if (nt > 0) body(0, std::integral_constant<int, 0>{}, std::true_type{});
  for (int t = 1; t < nt; t += 3) {
    body(t, std::integral_constant<int, 1>{}, no{});
    if (t + 1 < nt) body(t + 1, std::integral_constant<int, 2>{}, no{});
    if (t + 2 < nt) body(t + 2, std::integral_constant<int, 0>{}, no{});
  }
  // P*V of the last tile; the early waves then wait at the barrier that
  // evens the counts.
  if (nt >= 1 && nt - 1 < wave_nt) {
    const uint32_t blast = ((nt - 1) % NST) * SB;
    if constexpr (D == 256) {  // vpre holds V^T 0, K 0, V^T 1, K 1
      vpre[1] = vpre[2];
      vpre[2] = vfrag(blast, 2);
    }
    __builtin_amdgcn_s_setprio(1);
    pv(blast, []() {});
    __builtin_amdgcn_s_setprio(0);
  }
  if (!late) barrier();

  const rsrc_t ro = make_rsrc(O + qhead, q_bytes);
  const rsrc_t rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int qi = qw + 32 * b + col;
    const float total = swap_halves_add(l_run[b]);
    const float inv = total > 0.f ? 1.0f / total : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (E)(oacc[b][db][4 * r + e] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), ro,
                                              (int)((qi * D + 32 * db + 8 * r + 4 * half) * 2),
                                              0, 0);
      }
    }
    if (half == 0) {
      const float lse = total > 0.f ? (m_run[b] + log2f(total)) * kLn2 : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qi * 4, 0, 0);
    }
  }
}

// ------------------------------------------------------------- host side --

struct Shape {
  int grid, block, lds, block_m, block_n, nq;
  int qb, nw;  // 32-query blocks per wave, waves per workgroup
};

template <int D>
void tile_info(Shape* sh) {
  sh->lds = Tile<kLayoutD<D>, kBlockN<D>>::LDS_BYTES;  // the same for every NW
  sh->block_n = kBlockN<D>;
}

constexpr int64_t kCUs = 256;  // gfx950 parts have 256 CUs
// LDS of the ping-pong kernel: three stages of 8 KiB of K and 8 KiB of V
// (of 16 KiB each at d = 256).
constexpr int kPingPongLds = 3 * 2 * 8192;

// The workgroup shape at d = 128: the largest whose grid still gives every CU
// two workgroups' worth of rows (512-row workgroups: two rounds of one per
// CU; 256-row ones: one round of two per CU), else 128 rows.
void pick_shape_128(int64_t BH, int Nq, int* qb, int* nw) {
  auto grid = [&](int rows) { return BH * (((int64_t)Nq + rows - 1) / rows); };
  if (grid(512) >= 2 * kCUs) {
    *qb = 2, *nw = 8;
  } else if (grid(256) >= 2 * kCUs) {
    *qb = 2, *nw = 4;
  } else {
    *qb = 1, *nw = 4;
  }
}

// d = 64: the ping-pong kernel's 512-row workgroups when both axes have at
// least 4096 rows and the grid gives every CU two of them, else 128 rows.
// On shorter rows the 512-row workgroups lost (-9% on causal B=8 H=16
// N=2048), on long ones they won (+5.1% on B=16 H=16 N=4096, +7.5% on the
// long causal shape at d = 64; interleaved A/B, bit-identical outputs).
void pick_shape_64(int64_t BH, int Nq, int Nk, int* qb, int* nw) {
  if (Nq >= 4096 && Nk >= 4096 && BH * (((int64_t)Nq + 511) / 512) >= 2 * kCUs) *qb = 2, *nw = 8;
}

// d = 96: the ping-pong kernel's 512-row workgroups when the grid gives every
// CU two of them, else one block a wave.
void pick_shape_96(int64_t BH, int Nq, int* qb, int* nw) {
  if (BH * (((int64_t)Nq + 511) / 512) >= 2 * kCUs) *qb = 2, *nw = 8;
}

// d = 32 and 256 (one block a wave): eight-wave workgroups (256 rows) when
// the grid gives two full rounds of them (two per CU at d = 32, one at
// d = 256), else four waves.
int pick_waves_one_block(int64_t BH, int Nq, int d) {
  const int64_t per_round = (d == 256 ? 1 : 2) * kCUs;
  return BH * (((int64_t)Nq + 255) / 256) >= 2 * per_round ? 8 : 4;
}

// Sizes shared by every entry point; Nk only bounds the key tensors.
int check_sizes(int B, int H, int Nq, int Nk, int d, Shape* sh) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return ATTN_ERR_HEADDIM;
  // One head's tensors are addressed with 32-bit byte offsets (plus one tile).
  if ((int64_t)Nq * d * 2 + (int64_t)kBlockMMax * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
  if ((int64_t)Nk * d * 2 + (int64_t)128 * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
  if ((int64_t)B * H > INT32_MAX) return ATTN_ERR_SHAPE;
  switch (d) {
    case 32: tile_info<32>(sh); break;
    case 64: tile_info<64>(sh); break;
    case 96: tile_info<96>(sh); break;
    case 128: tile_info<128>(sh); break;
    default: tile_info<256>(sh); break;
  }
  sh->qb = 1, sh->nw = kWaves;
  if (d == 128) pick_shape_128((int64_t)B * H, Nq, &sh->qb, &sh->nw);
  if (d == 64) pick_shape_64((int64_t)B * H, Nq, Nk, &sh->qb, &sh->nw);
  if (d == 32 || d == 256) sh->nw = pick_waves_one_block((int64_t)B * H, Nq, d);
  if (d == 96) pick_shape_96((int64_t)B * H, Nq, &sh->qb, &sh->nw);
  sh->block = 64 * sh->nw;
  sh->block_m = 32 * sh->nw * sh->qb;
  if ((d == 64 || d == 96 || d == 128) && sh->qb == 2 && sh->nw == 8) sh->lds = kPingPongLds;
  if (d == 256 && sh->nw == 8) sh->lds = 2 * kPingPongLds;
  const int64_t nq = ((int64_t)Nq + sh->block_m - 1) / sh->block_m;
  const int64_t grid = (int64_t)B * H * nq;
  if (grid > INT32_MAX) return ATTN_ERR_SHAPE;
  sh->grid = (int)grid;
  sh->nq = (int)nq;
  return ATTN_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Args {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int BH, Nq, Nk;
  float c;
  hipStream_t stream;
};

template <typename E, int D, bool CAUSAL>
hipError_t launch_pp(const Shape& sh, const Args& a) {
  const E* qp = static_cast<const E*>(a.q);
  const E* kp = static_cast<const E*>(a.k);
  const E* vp = static_cast<const E*>(a.v);
  E* op = static_cast<E*>(a.o);
  float* lp = a.lse;
  int BH = a.BH, Nq = a.Nq, Nk = a.Nk, nq = sh.nq;
  float c = a.c;
  void* args[] = {&qp, &kp, &vp, &op, &lp, &BH, &Nq, &Nk, &nq, &c};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_pp_kernel<E, D, CAUSAL>),
                         dim3(sh.grid), dim3(sh.block), args, 0, a.stream);
}

template <typename E, int D, bool CAUSAL, int QB, int NW>
hipError_t launch(const Shape& sh, const Args& a) {
  const E* qp = static_cast<const E*>(a.q);
  const E* kp = static_cast<const E*>(a.k);
  const E* vp = static_cast<const E*>(a.v);
  E* op = static_cast<E*>(a.o);
  float* lp = a.lse;
  int BH = a.BH, Nq = a.Nq, Nk = a.Nk, nq = sh.nq;
  float c = a.c;
  void* args[] = {&qp, &kp, &vp, &op, &lp, &BH, &Nq, &Nk, &nq, &c};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<E, D, CAUSAL, QB, NW>),
                         dim3(sh.grid), dim3(sh.block), args, 0, a.stream);
}

template <typename E, int D, bool CAUSAL>
hipError_t launch_shape(const Shape& sh, const Args& a) {
  if constexpr (D == 256) {
    if (sh.nw == 8) return launch_pp<E, D, CAUSAL>(sh, a);
  }
  if constexpr (D == 96) {
    if (sh.qb == 2 && sh.nw == 8) return launch_pp<E, D, CAUSAL>(sh, a);
  }
  if constexpr (D == 32) {
    if (sh.nw == 8) return launch<E, D, CAUSAL, 1, 8>(sh, a);
  }
  if constexpr (D == 64 || D == 128) {
    if (sh.qb == 2 && sh.nw == 8) return launch_pp<E, D, CAUSAL>(sh, a);
  }
  if constexpr (D == 128) {
    if (sh.qb == 2) return launch<E, D, CAUSAL, 2, 4>(sh, a);
  }
  return launch<E, D, CAUSAL, 1, kWaves>(sh, a);
}

template <typename E>
hipError_t launch_type(const Shape& sh, const Args& a, int d, bool causal) {
  switch (d) {
    case 32: return causal ? launch_shape<E, 32, true>(sh, a) : launch_shape<E, 32, false>(sh, a);
    case 64: return causal ? launch_shape<E, 64, true>(sh, a) : launch_shape<E, 64, false>(sh, a);
    case 96: return causal ? launch_shape<E, 96, true>(sh, a) : launch_shape<E, 96, false>(sh, a);
    case 128:
      return causal ? launch_shape<E, 128, true>(sh, a) : launch_shape<E, 128, false>(sh, a);
    default:
      return causal ? launch_shape<E, 256, true>(sh, a) : launch_shape<E, 256, false>(sh, a);
  }
}

// Validation and launch behind every attention entry point.
int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
        int Nq, int Nk, int d, int dtype, float scale, int causal, void* stream) {
  Shape sh;
  const int rc = check_sizes(B, H, Nq, Nk, d, &sh);
  if (rc != ATTN_OK) return rc;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_DTYPE;
  uint32_t sbits;
  memcpy(&sbits, &scale, 4);
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_ERR_SCALE;  // NaN or +-inf
  if (sh.grid == 0) return ATTN_OK;  // B*H*Nq == 0: nothing to compute
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
  const size_t qbytes = (size_t)B * H * Nq * d * 2;
  const size_t kbytes = (size_t)B * H * Nk * d * 2;
  const size_t lbytes = (size_t)B * H * Nq * 4;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) ||
      overlaps(o, qbytes, v, kbytes) || overlaps(lse, lbytes, q, qbytes) ||
      overlaps(lse, lbytes, k, kbytes) || overlaps(lse, lbytes, v, kbytes) ||
      overlaps(lse, lbytes, o, qbytes))
    return ATTN_ERR_ALIAS;

  const Args a{q, k, v, o, lse, B * H, Nq, Nk, scale * kLog2e,
               static_cast<hipStream_t>(stream)};
  const hipError_t err = dtype == ATTN_BF16 ? launch_type<__bf16>(sh, a, d, causal != 0)
                                            : launch_type<_Float16>(sh, a, d, causal != 0);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal,
                        void* stream) {
  return run(q, k, v, o, lse, B, H, N, N, d, ATTN_BF16, scale, causal, stream);
}

extern "C" int attn_fwd_cross(const void* q, const void* k, const void* v, void* o,
                              float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                              int causal, void* stream) {
  return run(q, k, v, o, lse, B, H, Nq, Nk, d, ATTN_BF16, scale, causal, stream);
}

extern "C" int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, int dtype, float scale,
                           int causal, void* stream) {
  return run(q, k, v, o, lse, B, H, Nq, Nk, d, dtype, scale, causal, stream);
}

extern "C" const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid shape: sizes must be >= 0 and fit 32-bit head offsets";
    case ATTN_ERR_HEADDIM: return "unsupported head dimension: d must be 32, 64, 96, 128 or 256";
    case ATTN_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16 bytes, lse 4 bytes";
    case ATTN_ERR_ALIAS: return "output buffer overlaps an input or the other output";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_DTYPE: return "unsupported element type: ATTN_BF16 or ATTN_F16";
    case ATTN_ERR_SCRATCH: return "attn_bwd_noalloc: B*H*Nq exceeds its static buffer (4194304 rows)";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_launch_shape(int B, int H, int N, int d, int causal, int* grid,
                                     int* block, int* lds_bytes, int* block_m,
                                     int* block_n) {
  (void)causal;
  if (!grid || !block || !lds_bytes || !block_m || !block_n) return ATTN_ERR_NULL;
  Shape sh;
  const int rc = check_sizes(B, H, N, N, d, &sh);
  if (rc != ATTN_OK) return rc;
  *grid = sh.grid;
  *block = sh.block;
  *lds_bytes = sh.lds;
  *block_m = sh.block_m;
  *block_n = sh.block_n;
  return ATTN_OK;
}
