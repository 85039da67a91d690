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
// Design for MI355X (gfx950): one workgroup of 4 waves owns 128 query rows of
// one (batch, head); each wave owns 32 rows. Key/value tiles of 8192 elements
// (64 keys at d=128, 128 keys at d=64) are streamed HBM -> registers -> LDS,
// double buffered, one tile ahead. Both contractions run on
// v_mfma_f32_32x32x16_bf16:
//
//   S^T (keys x queries) = K (keys x d) * Q^T (d x queries)
//   O^T (d x queries)   += V^T (d x keys) * P^T (keys x queries)
//
// Computing the transposed products puts one query per lane (lane % 32) in
// both accumulators, so the row statistics (max, sum, rescale) are per-lane
// scalars plus one exchange between the two 32-lane halves, and the S^T
// accumulator, rounded to bf16, is already the B operand of the P*V product
// after a fixed permutation of the key order inside each 16-key slice. V^T is
// written to LDS in that permuted order, so the A operand is one 16-byte LDS
// read per lane.
//
// MFMA 32x32x16 fragment layout used below (lane l, h = l / 32, c = l % 32):
//   A (32 x 16):  lane holds row c, k-elements 8h .. 8h+7
//   B (16 x 32):  lane holds column c, k-elements 8h .. 8h+7
//   C (32 x 32):  register i holds row 8*(i/4) + 4h + i%4, column c
// A and B agree on which k each (h, element) carries, so any hardware k order
// gives the same contraction.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mi_attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;     // threads per workgroup
constexpr int kBlockM = 32 * kWaves;      // query rows per workgroup

// Per head dimension D: the key tile and its LDS layout.
template <int D>
struct Tile {
  static constexpr int BN = 8192 / D;          // keys per step (64 or 128)
  static constexpr int NKB = BN / 32;          // 32-key MFMA blocks per step
  static constexpr int KSTRIDE = D + 8;        // K row pitch in LDS (bf16), 16 B pad
  static constexpr int K_ELEMS = BN * KSTRIDE; // K tile
  static constexpr int VT_ELEMS = D * BN;      // V^T tile
  static constexpr int STAGE = K_ELEMS + VT_ELEMS;
  static constexpr int CPR = D / 8;            // 16-byte chunks per global row
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static_assert(BN * CPR == 4 * kThreads, "each thread stages 4 chunks of K and of V");
};

// Key order inside a 16-key slice of V^T in LDS: swaps bits 2 and 3 of the
// key offset, matching where the S^T accumulator leaves each key (C layout
// row 8*(i/4) + 4h + i%4 read as B-operand element 8h + j).
__device__ __forceinline__ int slice_pos(int o) {
  return (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

// XOR swizzle of 16-byte blocks inside a V^T row, so that the 8 rows read by
// 8 consecutive lanes land in 8 different blocks (distinct banks) and the
// transposing writes spread over blocks too.
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Workgroup id -> (batch*head, query tile). Workgroups are dealt to the 8
// XCDs round-robin, so when B*H is a multiple of 8 each XCD gets the heads
// h = x (mod 8) and walks them head by head (non-causal: the q-tiles of one
// head run together and share that XCD's L2 for K and V) or q-tile by q-tile
// from the heaviest (causal: longest key prefix first, so short tiles fill the
// tail).
__device__ __forceinline__ void map_block(int bid, int BH, int nq, bool causal,
                                          int& bh, int& qt) {
  if ((BH & 7) == 0) {
    const int x = bid & 7, j = bid >> 3, hpx = BH >> 3;
    if (causal) {
      qt = nq - 1 - j / hpx;
      bh = x + 8 * (j % hpx);
    } else {
      bh = x + 8 * (j / nq);
      qt = j % nq;
    }
  } else if (causal) {
    qt = nq - 1 - bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / nq;
    qt = bid % nq;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, __bf16* __restrict__ O,
    float* __restrict__ LSE, int BH, int N, int nq, float c) {
  using T = Tile<D>;
  constexpr int BN = T::BN, NKB = T::NKB, KS = T::KSTRIDE, CPR = T::CPR;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;

  int bh, qt;
  map_block(blockIdx.x, BH, nq, CAUSAL, bh, qt);
  const int q0 = qt * kBlockM;
  const int qw = q0 + 32 * wave;  // first query row of this wave
  const int qi = qw + col;        // this lane's query row

  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = Q + head;
  const __bf16* Kh = K + head;
  const __bf16* Vh = V + head;

  // Q^T fragments (B operand): lane holds Q[qi][16s + 8h .. +7] for s < D/16.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (qi < N) {
      qf[s] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qi * D + 16 * s + 8 * half);
    } else {
      qf[s] = bf16x8{};
    }
  }

  // Keys this workgroup / this wave can see.
  const int kv_end = CAUSAL ? min(N, q0 + kBlockM) : N;
  const int wave_kv_end = CAUSAL ? min(N, qw + 32) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  // Staging: thread owns rows kr .. kr+3 of the tile, 16-byte chunk dc.
  const int kr = 4 * (tid / CPR);
  const int dc = tid % CPR;
  u32x4 kreg[4], vreg[4];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = k0 + kr + i;
      if (row < N) {
        const size_t off = (size_t)row * D + 8 * dc;
        kreg[i] = *reinterpret_cast<const u32x4*>(Kh + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vh + off);
      } else {  // past the end: zeros (their weight is 0, and 0 * 0 stays finite)
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int stage) {
    __bf16* Ks = smem + stage * T::STAGE;
    __bf16* Vts = Ks + T::K_ELEMS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(Ks + (kr + i) * KS + 8 * dc) = kreg[i];
    }
    // V^T: for each of the chunk's 8 columns d, the 4 keys kr..kr+3 are
    // contiguous in the permuted slice order -> one 8-byte write per column.
    const int pos = 16 * (kr >> 4) + slice_pos(kr & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      uint32_t lo, hi;
      if (e & 1) {
        lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
        hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
      } else {
        lo = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
        hi = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
      }
      const int d = 8 * dc + e;
      const int blk = (pos >> 3) ^ vt_swz(d);
      *reinterpret_cast<u32x2*>(Vts + d * BN + blk * 8 + (pos & 7)) = u32x2{lo, hi};
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float run_max = -INFINITY;  // in log2 units: max of s * scale * log2(e)
  float run_sum = 0.f;        // this lane's share of the row sum

  const bool pos_scale = c >= 0.f;
  const float mask_val = pos_scale ? -INFINITY : INFINITY;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    if (t + 1 < ntiles) load_tile(k0 + BN);

    if (k0 < wave_kv_end) {
      const __bf16* Ks = smem + (t & 1) * T::STAGE;
      const __bf16* Vts = Ks + T::K_ELEMS;

      // S^T = K * Q^T for the tile's NKB blocks of 32 keys.
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              Ks + (32 * kb + col) * KS + 16 * s + 8 * half);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }

      // Hide keys past the end and (causal) keys after the query.
      const bool need_mask = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
            const bool vis = key < N && (!CAUSAL || key <= qi);
            if (!vis) sacc[kb][i] = mask_val;
          }
        }
      }

      // Row extreme of the raw scores (max if the scale is >= 0, else min),
      // combined across the two lane halves that share the query.
      float ext = sacc[0][0];
      if (pos_scale) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) ext = fmaxf(ext, sacc[kb][i]);
        ext = fmaxf(ext, __shfl_xor(ext, 32));
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) ext = fminf(ext, sacc[kb][i]);
        ext = fminf(ext, __shfl_xor(ext, 32));
      }
      // fmaxf ignores a NaN from 0 * inf (scale 0, row fully masked here).
      const float new_max = fmaxf(run_max, ext * c);
      const float alpha = __builtin_amdgcn_exp2f(run_max - new_max);

      // p = 2^(s*c - m): the exp of the scaled, max-subtracted score.
      float tile_sum = 0.f;
      bf16x8 pb[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, -new_max));
          if (need_mask && sacc[kb][i] == mask_val) p = 0.f;
          tile_sum += p;
          pb[kb][i >> 3][i & 7] = (__bf16)p;
        }
      }
      run_sum = run_sum * alpha + tile_sum;
      run_max = new_max;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

      // O^T += V^T * P^T, 16 keys per MFMA.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
          const int g = 2 * kb + sg;  // 16-key slice index in the tile
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + col;
            const int blk = (2 * g + half) ^ vt_swz(d);
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vts + d * BN + blk * 8);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][sg], oacc[db], 0, 0, 0);
          }
        }
      }
    }

    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l (bf16), lse = (m + log2 l) * ln 2.
  const float total = run_sum + __shfl_xor(run_sum, 32);
  if (qi < N) {
    const float inv = 1.0f / total;
    __bf16* Orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(oacc[db][4 * r + e] * inv);
        *reinterpret_cast<bf16x4*>(Orow + 32 * db + 8 * r + 4 * half) = v4;
      }
    }
    if (half == 0) LSE[(size_t)bh * N + qi] = (run_max + log2f(total)) * kLn2;
  }
}

// ------------------------------------------------------------- host side --

struct Shape {
  int grid, block, lds, block_m, block_n, nq;
};

int check_sizes(int B, int H, int N, int d, Shape* sh) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  const int64_t rows = (int64_t)B * H * N;
  if (rows > 0 && rows > INT64_MAX / d) return ATTN_ERR_SHAPE;
  if ((int64_t)B * H > INT32_MAX) return ATTN_ERR_SHAPE;
  const int64_t nq = ((int64_t)N + kBlockM - 1) / kBlockM;
  const int64_t grid = (int64_t)B * H * nq;
  if (grid > INT32_MAX) return ATTN_ERR_SHAPE;
  sh->grid = (int)grid;
  sh->block = kThreads;
  sh->lds = d == 64 ? Tile<64>::LDS_BYTES : Tile<128>::LDS_BYTES;
  sh->block_m = kBlockM;
  sh->block_n = d == 64 ? Tile<64>::BN : Tile<128>::BN;
  sh->nq = (int)nq;
  return ATTN_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

template <int D, bool CAUSAL>
hipError_t launch(const Shape& sh, const void* q, const void* k, const void* v, void* o,
                  float* lse, int BH, int N, float c, hipStream_t stream) {
  const __bf16* qp = static_cast<const __bf16*>(q);
  const __bf16* kp = static_cast<const __bf16*>(k);
  const __bf16* vp = static_cast<const __bf16*>(v);
  __bf16* op = static_cast<__bf16*>(o);
  int nq = sh.nq;
  void* args[] = {&qp, &kp, &vp, &op, &lse, &BH, &N, &nq, &c};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<D, CAUSAL>),
                         dim3(sh.grid), dim3(sh.block), args, 0, stream);
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, float scale, int causal,
                        void* stream) {
  Shape sh;
  const int rc = check_sizes(B, H, N, d, &sh);
  if (rc != ATTN_OK) return rc;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  if (sh.grid == 0) return ATTN_OK;  // B*H*N == 0: nothing to compute
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
  const size_t tbytes = (size_t)B * H * N * d * 2;
  const size_t lbytes = (size_t)B * H * N * 4;
  if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
      overlaps(o, tbytes, v, tbytes) || overlaps(lse, lbytes, q, tbytes) ||
      overlaps(lse, lbytes, k, tbytes) || overlaps(lse, lbytes, v, tbytes) ||
      overlaps(lse, lbytes, o, tbytes))
    return ATTN_ERR_ALIAS;

  const float c = scale * kLog2e;
  const int BH = B * H;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (d == 64) {
    err = causal ? launch<64, true>(sh, q, k, v, o, lse, BH, N, c, st)
                 : launch<64, false>(sh, q, k, v, o, lse, BH, N, c, st);
  } else {
    err = causal ? launch<128, true>(sh, q, k, v, o, lse, BH, N, c, st)
                 : launch<128, false>(sh, q, k, v, o, lse, BH, N, c, st);
  }
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid shape: B, H, N must be >= 0 and the sizes must fit";
    case ATTN_ERR_HEADDIM: return "unsupported head dimension: d must be 64 or 128";
    case ATTN_ERR_ALIGN: return "misaligned pointer: q, k, v, o need 16 bytes, lse 4 bytes";
    case ATTN_ERR_ALIAS: return "output buffer overlaps an input or the other output";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_launch_shape(int B, int H, int N, int d, int causal, int* grid,
                                     int* block, int* lds_bytes, int* block_m,
                                     int* block_n) {
  (void)causal;
  if (!grid || !block || !lds_bytes || !block_m || !block_n) return ATTN_ERR_NULL;
  Shape sh;
  const int rc = check_sizes(B, H, N, d, &sh);
  if (rc != ATTN_OK) return rc;
  *grid = sh.grid;
  *block = sh.block;
  *lds_bytes = sh.lds;
  *block_m = sh.block_m;
  *block_n = sh.block_n;
  return ATTN_OK;
}
