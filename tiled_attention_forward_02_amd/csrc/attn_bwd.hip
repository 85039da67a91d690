// attn_bwd.hip - attention backward (dQ, dK, dV) for gfx950 (CDNA4) and its C ABI.
//
// The gradients of the fused attention forward ("[GPU] Deep Learning for HPC",
// section "Flash Attention"; scale and causal flag as in the Triton forward
// signature on null-ptr.tistory.com, category "development") for an upstream
// gradient dO of O. The pages print no backward; it is the chain rule of the
// forward definition: with P the softmax weights,
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_c dO_ic O_ic,
//   dQ = scale dS K,  dK = scale dS^T Q,
//
// where D_i equals sum_j P_ij dP_ij (the softmax Jacobian's row term) because
// O = P V. P is never stored: it is recomputed tile by tile from the scores
// and the forward's log-sum-exp, P = 2^(s*scale*log2(e) - lse*log2(e)).
//
// Kernels on the caller's stream, no atomics, every output written once:
//
//  * dQ kernel: one workgroup per 128 (or 256) query rows of one head (a query per
//    lane, as in the forward), keys streamed through LDS in tiles. It also
//    forms D_i from its own rows of O and dO and writes it to `delta`.
//      S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T * (dP^T - D),  dQ^T += K^T dS^T
//  * key-side kernel: one workgroup per 128 (or 256) keys (a key per lane), query
//    tiles streamed through LDS in two row-major copies (row reads and
//    transposing reads); one pass accumulates both gradients.
//      S = Q K^T,  dP = dO V^T,  dS = P * (dP - D),
//      dV^T += dO^T P,  dK^T += Q^T dS
//
// In both, the C accumulator of P or dS, rounded to the input type, is the B
// operand of the next product once the rows inside each 16-row slice follow
// slice_pos(). The matching transposed A operands (K^T, Q^T, dO^T) come from
// transposing LDS reads of a row-major copy of the tile, which hand each
// lane 4 rows of one column in that order. Masked
// entries (causal, and keys past Nk in the dQ kernel) get P = 0 by a select
// after the exponent, so any finite scale works, 0 and negative included.
// A row with lse = -inf (no visible key) gets P = 0 throughout.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "attn_bwd_kernels.h"
#include "common.h"
#include "mi_attn.h"

namespace {

using namespace mi_attn;

// ------------------------------------------------------------- host side --

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}


constexpr int64_t kCUs = 256;  // gfx950 parts have 256 CUs

// Waves per workgroup (both kernels): eight at d = 128 without the causal
// mask when both axes have at least 2048 rows, both grids give two rounds of
// one eight-wave workgroup per CU and the offsets of one such workgroup past
// the end stay within 32 bits, else four.
int pick_waves(int64_t BH, int Nq, int Nk, int d, bool causal) {
  if (d != 128 || causal || Nq < 2048 || Nk < 2048) return 4;
  auto grid = [&](int n) { return BH * (((int64_t)n + 255) / 256); };
  if (grid(Nq) < 2 * kCUs || grid(Nk) < 2 * kCUs) return 4;
  if ((int64_t)(Nq > Nk ? Nq : Nk) * d * 2 + (int64_t)256 * d * 2 > INT32_MAX) return 4;
  return 8;
}

// The dQ kernel at d = 128 runs the ping-pong form (256 queries a
// workgroup) with the eight-wave shape, and with the causal mask under the
// same size conditions on the query side (the key-side kernel then keeps
// four waves, which lost less there).
bool pick_dq_pp(int64_t BH, int Nq, int Nk, int d, bool causal, int nw) {
  if (d != 128) return false;
  if (!causal) return nw == 8;
  if (Nq < 2048 || Nk < 2048 || BH * (((int64_t)Nq + 255) / 256) < 2 * kCUs) return false;
  return (int64_t)(Nq > Nk ? Nq : Nk) * d * 2 + (int64_t)256 * d * 2 <= INT32_MAX;
}

template <typename E>
hipError_t launch_bwd_type(const BwdArgs& a, int d, bool causal) {
  switch (d) {
    case 32: return causal ? launch_bwd<E, 32, true, 4>(a) : launch_bwd<E, 32, false, 4>(a);
    case 64: return causal ? launch_bwd<E, 64, true, 4>(a) : launch_bwd<E, 64, false, 4>(a);
    case 96: return causal ? launch_bwd<E, 96, true, 4>(a) : launch_bwd<E, 96, false, 4>(a);
    default:
      if (causal) return launch_bwd<E, 128, true, 4>(a);
      return a.nw == 8 ? launch_bwd<E, 128, false, 8>(a) : launch_bwd<E, 128, false, 4>(a);
  }
}

// ----------------------------------------------------- static scratch --

// Row sums D for attn_bwd_noalloc, in a static device array instead of a
// caller buffer: kScratchRows floats (16 MiB) on each device the library
// runs on, held until the process ends. Host code never uses the array's
// name as an address (on the host it is only a stand-in); it asks the runtime
// for the device address once per device and passes that to the kernels.
constexpr int64_t kScratchRows = int64_t(1) << 22;  // B * H * Nq at most

}  // namespace

static __device__ __align__(256) float scratch[kScratchRows];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_at[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current); NULL if the runtime cannot give it.
float* scratch_rows() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_at[dev] = static_cast<float*>(ptr);
  }
  return g_scratch_at[dev];
}

// Validation and launch behind both backward entry points. With use_scratch
// the row sums D go to the library's own buffer (`delta` is ignored), so no
// caller buffer needs to be checked for them.
int bwd_run(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* d_o, void* dq, void* dk, void* dv, float* delta, bool use_scratch, int B,
            int H, int Nq, int Nk, int d, int dtype, float scale, int causal, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return ATTN_ERR_HEADDIM;
  if ((int64_t)Nq * d * 2 + (int64_t)kBlockRows * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
  if ((int64_t)Nk * d * 2 + (int64_t)kBlockRows * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
  const int64_t BH = (int64_t)B * H;
  const int nw = pick_waves(BH, Nq, Nk, d, causal != 0);
  const bool dq_pp = pick_dq_pp(BH, Nq, Nk, d, causal != 0, nw);
  const int64_t rows = 32 * nw, qrows = dq_pp ? 256 : rows;
  const int64_t nq = ((int64_t)Nq + qrows - 1) / qrows;
  const int64_t nk = ((int64_t)Nk + rows - 1) / rows;
  if (BH * nq > INT32_MAX || BH * nk > INT32_MAX) return ATTN_ERR_SHAPE;
  if (use_scratch && BH * Nq > kScratchRows) return ATTN_ERR_SCRATCH;
  if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_DTYPE;
  uint32_t sbits;
  memcpy(&sbits, &scale, 4);
  if ((sbits & 0x7f800000u) == 0x7f800000u) return ATTN_ERR_SCALE;
  if (BH == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  if (Nq > 0 && (!q || !o || !lse || !d_o || !dq || (!use_scratch && !delta))) return ATTN_ERR_NULL;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)d_o |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15)
    return ATTN_ERR_ALIGN;
  if (((uintptr_t)lse | (use_scratch ? 0 : (uintptr_t)delta)) & 3) return ATTN_ERR_ALIGN;
  const size_t qb = (size_t)BH * Nq * d * 2, kb = (size_t)BH * Nk * d * 2;
  const size_t lb = (size_t)BH * Nq * 4;
  const struct {
    const void* p;
    size_t n;
  } in[] = {{q, qb}, {k, kb}, {v, kb}, {o, qb}, {lse, lb}, {d_o, qb}},
    out[] = {{dq, qb}, {dk, kb}, {dv, kb}, {use_scratch ? nullptr : delta, lb}};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i].p, out[i].n, in[j].p, in[j].n)) return ATTN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(out[i].p, out[i].n, out[j].p, out[j].n)) return ATTN_ERR_ALIAS;
  }
  if (use_scratch && Nq > 0) {
    delta = scratch_rows();
    if (!delta) return ATTN_ERR_LAUNCH;
  }

  const BwdArgs a{q, k, v, o, d_o, lse, dq, dk, dv, delta, (int)BH, Nq, Nk, (int)nq, (int)nk,
                  nw, dq_pp, scale * kLog2e, scale, static_cast<hipStream_t>(stream)};
  const hipError_t err = d == 256 ? launch_bwd_d256(a, causal != 0, dtype == ATTN_F16)
                         : dtype == ATTN_BF16 ? launch_bwd_type<__bf16>(a, d, causal != 0)
                                              : launch_bwd_type<_Float16>(a, d, causal != 0);
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                        float* delta, int B, int H, int Nq, int Nk, int d, int dtype,
                        float scale, int causal, void* stream) {
  return bwd_run(q, k, v, o, lse, d_o, dq, dk, dv, delta, false, B, H, Nq, Nk, d, dtype, scale,
                 causal, stream);
}

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                                int B, int H, int Nq, int Nk, int d, int dtype, float scale,
                                int causal, void* stream) {
  return bwd_run(q, k, v, o, lse, d_o, dq, dk, dv, nullptr, true, B, H, Nq, Nk, d, dtype, scale,
                 causal, stream);
}
