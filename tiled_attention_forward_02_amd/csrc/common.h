// common.h - device helpers shared by the attention forward and backward
// kernels for gfx950 (CDNA4): element types and their MFMA, buffer resources,
// LDS DMA of row-major tiles, transposing LDS reads and their row pitch,
// lane-half exchange, the key order inside a 16-key slice and the workgroup
// -> tile mapping.
//
// MFMA 32x32x16 fragment layout used throughout (lane l, h = l / 32, c = l % 32):
//   A (32 x 16):  lane holds row c, k-elements 8h .. 8h+7
//   B (16 x 32):  lane holds column c, k-elements 8h .. 8h+7
//   C (32 x 32):  register i holds row 8*(i/4) + 4h + i%4, column c
// A and B agree on which k each (h, element) carries, so any hardware k order
// gives the same contraction.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

namespace mi_attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// The two 16-bit input types: 8-element MFMA operands, the 32x32x16 MFMA
// with fp32 accumulation, and rounding from fp32 (to nearest even).
template <typename E>
struct Elem;
template <>
struct Elem<__bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Elem<_Float16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kWaves = 4;              // waves per workgroup
constexpr int kThreads = 64 * kWaves;  // threads per workgroup

// Key order inside a 16-key slice of a transposed tile in LDS: swaps bits 2
// and 3 of the offset, matching where a C accumulator leaves each row (C
// layout row 8*(i/4) + 4h + i%4 read as B-operand element 8h + j). Its own
// inverse.
__device__ __forceinline__ int slice_pos(int o) {
  return (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

// Workgroup id -> (batch*head, tile). Workgroups are dealt to the 8 XCDs
// round-robin, so when B*H is a multiple of 8 each XCD gets the heads
// h = x (mod 8) and walks them head by head (not heaviest_first: the tiles of
// one head run together and share that XCD's L2) or tile by tile from the
// last index down (heaviest_first: the caller numbers tiles so that the last
// is the heaviest; short tiles fill the tail).
__device__ __forceinline__ void map_block(int bid, int BH, int nt, bool heaviest_first,
                                          int& bh, int& t) {
  if ((BH & 7) == 0) {
    const int x = bid & 7, j = bid >> 3, hpx = BH >> 3;
    if (heaviest_first) {
      t = nt - 1 - j / hpx;
      bh = x + 8 * (j % hpx);
    } else {
      bh = x + 8 * (j / nt);
      t = j % nt;
    }
  } else if (heaviest_first) {
    t = nt - 1 - bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / nt;
    t = bid % nt;
  }
}

// Buffer resource over [base, base + bytes): loads past the end return 0 and
// stores past the end are dropped by the hardware range check.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

// A byte in LDS, addressed as such (a generic pointer cast to LDS needs a
// null check at each use).
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ lds_char* to_lds(void* shared_array) {
  return (lds_char*)shared_array;
}

// 16 bytes per lane from the buffer at byte_off straight into LDS, no
// registers: the wave's 64 lanes fill the 1024 bytes at lds_base in lane
// order (lane l at lds_base + 16 l); an offset past the buffer writes zeros
// without a fetch. Completion is counted by vmcnt, like any buffer load.
__device__ __forceinline__ void load16_lds(rsrc_t r, lds_char* lds_base, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_base, 16, (int)byte_off, 0, 0, 0);
}

// LDS DMA of one row-major tile: the first BR rows of a [*, D] tensor (16-bit
// elements) that a buffer resource starts at, into BR rows of PITCH
// elements, PITCH / 8 16-byte slots a row of which D / 8 hold data.
// Instruction u of the tile (u = wave, wave + W, ...; W waves; whether u exists
// is a uniform branch) writes slots 64 u .. 64 u + 63, lane l slot
// 64 u + l; lanes of pad slots, of chunks past the data and past the tile
// get an offset beyond any buffer (zeros, no fetch). The instructions write
// SPAN bytes from the tile's start, a multiple of 1024 that the caller's
// layout reserves.
template <int D, int BR, int PITCH, int W = kWaves>
struct DmaTile {
  static constexpr int SLOTS = PITCH / 8;
  static constexpr int NINSTR = (BR * SLOTS + 63) / 64;
  static constexpr int NW = (NINSTR + W - 1) / W;  // per wave, at most
  static constexpr int SPAN = NINSTR * 1024;
  static constexpr uint32_t kNoFetch = 0x80000000u;  // > any head's bytes
  uint32_t off[NW];
  __device__ __forceinline__ DmaTile(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int slot = 64 * (wave + W * i) + lane;
      const int row = slot / SLOTS, ch = slot % SLOTS;
      off[i] = row < BR && ch < D / 8 ? (uint32_t)(row * D + 8 * ch) * 2 : kNoFetch;
    }
  }
  // r_tile's base is the tile's first row (its records counted from there):
  // the per-lane offsets are fixed, so placing a tile is scalar work. Rows
  // past the buffer's end are zero-filled by the range check.
  __device__ __forceinline__ void issue(rsrc_t r_tile, lds_char* tile, int wave) const {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int u = wave + W * i;
      if (u < NINSTR) load16_lds(r_tile, tile + 1024 * u, off[i]);
    }
  }
};

// Row pitch (elements) of a row-major tile read by lds_read_tr16, for layout
// head dimension DL. The 64-bank LDS serves 32 lanes of an 8-byte read at a
// time; those lanes cover 4 consecutive rows x 64 bytes, conflict-free when
// the rows start an odd multiple of 64 bytes apart (VS = 32 mod 64). At
// DL = 64 that pitch (96) would keep four workgroups from fitting in LDS; the
// forward lays d = 64 tiles out unpadded and swizzled instead, and 80 remains
// only this function's answer for it.
template <int DL>
constexpr int tr_pitch() {
  return DL == 64 ? 80 : (DL % 64 == 32 ? DL : DL + 32);
}

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16). Each lane gives
// the address of 4 consecutive elements (8 bytes). Within each group of 16
// lanes, lane 4a + b receives, as its element e, element b of the 4 given by
// lane a + 4e of the group (checked on gfx950 with a layout probe).
//
// `p` is restrict so that the read carries alias-scope metadata once inlined.
// Without it, the compiler puts a vmcnt(0) before every transposing read
// while any LDS DMA is in flight. That includes the DMA of a later tile into
// another stage, so a tile's P*V would wait for the next tile's loads. Plain
// LDS reads get no such wait, and neither now do these. Every kernel here
// orders its DMA'd tiles by its own vmcnt wait and barrier before any read.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* __restrict__ p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// -inf where `masked` has all bits set, x where it is 0: one v_bfi_b32. A
// bit select on a sign-extended difference needs no per-element lane mask
// (a compare would hold one SGPR pair per element of a tile until its
// select, more than the SGPR file at 64 elements).
__device__ __forceinline__ float neg_inf_where(int masked, float x) {
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(masked), "s"(-INFINITY), "v"(x));
  return r;
}

// Byte offset, within a row-major tile of pitch TS, of this lane's address
// for lds_read_tr16 reads of the MFMA A operand of a 16-row slice: lane
// 16 g + s points at row 4 (g / 2) + s / 4, columns 16 (g % 2) + 4 (s % 4)
// .. +3, and then holds column lane % 32 of rows 4 h .. 4 h + 3 of the slice
// (h = lane / 32); a second read 8 rows further gives rows 8 + 4 h ..
// 8 + 4 h + 3. Those are the rows that the B operand's slots 0-7 carry
// (slice_pos order).
template <int TS>
__device__ __forceinline__ uint32_t tr_lane_off(int lane) {
  return (uint32_t)((4 * (lane >> 5) + ((lane & 15) >> 2)) * TS + 16 * ((lane >> 4) & 1) +
                    4 * (lane & 3)) * 2;
}

// The 8-element A operand of rows `row0` .. row0 + 15 (a 16-row slice) and
// columns `col0` .. col0 + 31 from a copy for transposing reads at `tile`.
template <typename V8, int TS>
__device__ __forceinline__ V8 tr_operand(const char* tile, uint32_t lane_off, int row0,
                                         int col0) {
  const char* p = tile + lane_off + (row0 * TS + col0) * 2;
  const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * TS * 2);
  return __builtin_bit_cast(V8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Value of x in the lane 32 positions away, combined with op (same result in
// both lanes of the pair, bit for bit).
__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mi_attn
