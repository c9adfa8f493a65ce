// LDS tiles of bf16 rows streamed in by DMA, and the MFMA operand reads on
// them (shared by the attention and the affine-recurrence kernels).
//
// Rows of D bf16 go from global memory into LDS with gfx950's LDS-DMA loads
// (buffer_load ... lds, 16 bytes per lane: lane l of one instruction fills
// bytes [16l, 16l + 16) of a 1 KB block), so no registers or VALU are spent
// staging them. Tiles stay row major, [row][column], with 16-byte chunks
// XOR-swizzled within a row instead of padded:
//   "K" layout: chunk c of row r sits at c ^ swz_k(r), so the 16 rows that a
//      quarter-wave reads for one MFMA operand (same logical chunk, one row
//      per lane) hit 16 bank groups, and so do the transposing reads of the
//      same tile (tr_offset_k);
//   "V" layout: chunk c of row r sits at c ^ swz_v(r), for operands whose
//      k index runs down the rows (rows of the tile = k, columns = the
//      operand's rows): they are read with ds_read_b64_tr_b16, which hands
//      lane j of a 16-lane group element (j % 4) of the 8-byte loads of lanes
//      4e + j/4, e = 0..3. If lane 4a + b of the group loads columns
//      [4b, 4b + 4) of row k0 + a, lane j receives X[k0 + e][j], e = 0..3:
//      four consecutive k of one column, as the fragment needs. The swizzle
//      spreads the 4 rows x 4 chunks a half-wave reads over the banks.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace infini {

// The K layout's swizzle serves three reads without bank conflicts: 16
// consecutive rows at one logical chunk (the row-wise operand loads: a
// bijection of r mod 16 onto the chunks, for d = 64 per row parity); the
// transposing reads of 4 rows x 4 chunks (rows 4k .. 4k + 3 get distinct
// values of swz >> 2 for d = 128, rows r and r + 2 distinct bit 2 for d = 64);
// and, for d = 128, two rows of 8 chunk pairs (rows r, r + 1 of opposite
// parity). It has period 16 in r.
template <int D> __device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? 4 * (r & 3) + (((r >> 2) & 3) ^ (r & 1))
                  : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int D> __device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ const bf16* lds_at(const bf16* base, uint32_t byte_off) {
  return reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Buffer resource over `bytes` bytes from `base` (raw, no stride; dword 3 as
// gfx9 wants it for untyped loads). Loads through it take the base from
// scalar registers and a 32-bit per-lane offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const bf16* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, (int)bytes, 0x00020000);
}

// The same 16-byte LDS-DMA load written as inline assembly. The compiler
// neither counts these loads nor inserts waits for them (with the builtin it
// must assume that any later LDS access, or the fence of a barrier, depends
// on every DMA load in flight), so a kernel that uses them waits for them
// explicitly (wait_vmcnt, s_waitcnt). Each sets M0, the instruction's LDS
// base, itself: a kernel must not mix them with the builtin, which expects
// M0 to be the compiler's.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 asm_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
__device__ __forceinline__ void dma16_asm(void* lds, u32x4 rsrc, uint32_t voff, uint32_t soff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

template <int D, int NW, int BN>
struct DmaTile {
  static constexpr int NT = NW * 64;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int CHUNKS = BN * CPR;            // per tile, per tensor
  static constexpr int PER_WAVE = CHUNKS / 64 / NW;  // DMA instructions per wave and tensor
  static_assert(CHUNKS % (64 * NW) == 0, "tile split");
  // Instruction j of wave w fills tile rows from (j NW + w) 64 / CPR on. When
  // the swizzles of those rows do not depend on j (NW a multiple of 4 for
  // d = 128, even for d = 64), instruction j's lane offsets are instruction
  // 0's plus J_STEP j bytes, which the load takes as a scalar offset.
  static constexpr bool J_INV = D == 128 ? NW % 4 == 0 : NW % 2 == 0;
  static constexpr uint32_t J_STEP = NW * (64 / CPR) * 2 * D;
  static constexpr int NOFF = J_INV ? 1 : PER_WAVE;
  // per lane: byte offset, from the tile's first row, of the 16-byte chunk
  // it fetches (the same tile row for K and V)
  uint32_t k_off[NOFF], v_off[NOFF];

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int j = 0; j < NOFF; ++j) {
      const int p = (j * NW + w) * 64 + lane;  // physical chunk of the tile
      const int r = p / CPR, phys = p % CPR;
      k_off[j] = 2 * (r * D + 8 * (phys ^ swz_k<D>(r)));
      v_off[j] = 2 * (r * D + 8 * (phys ^ swz_v<D>(r)));
    }
  }
  // Issue the loads of key tile k0 of one tensor (K if IS_K, else V) into
  // Xs ([BN][D]); w is the (wave-uniform) wave index. Each load is a
  // buffer_load ... lds of 16 bytes per lane from a resource over the tile's
  // rows. In a tail tile, rows past the segment's end repeat its last row
  // (finite; the causal mask removes them).
  template <bool IS_K>
  __device__ __forceinline__ void issue(const bf16* X, bf16* Xs, int k0, int n_s, int w) const {
    const uint32_t* off = IS_K ? k_off : v_off;
    const int rows = min(BN, n_s - k0);
    const __amdgpu_buffer_rsrc_t rx = raw_rsrc(X + (int64_t)k0 * D, (uint32_t)rows * D * 2);
    if (rows == BN) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int blk = (j * NW + w) * 64 * 8;  // element offset of this wave's 1 KB block
        const uint32_t sj = J_INV ? j * J_STEP : 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(Xs + blk), 16, off[J_INV ? 0 : j], sj, 0, 0);
      }
    } else {
      const uint32_t lim = (uint32_t)rows * (2 * D);  // bytes of the valid rows
      const uint32_t last = lim - 2 * D;              // start of the last valid row
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int blk = (j * NW + w) * 64 * 8;
        const uint32_t xj = J_INV ? off[0] + j * J_STEP : off[j];
        const uint32_t xo = xj < lim ? xj : last + (xj & (2 * D - 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(Xs + blk), 16, xo, 0, 0, 0);
      }
    }
  }
  // issue() for a tile known to hold BN rows of the segment: every lane's
  // offset is its fixed one plus a scalar step, with no clamping
  template <bool IS_K>
  __device__ __forceinline__ void issue_full(const bf16* X, bf16* Xs, int k0, int w) const {
    const uint32_t* off = IS_K ? k_off : v_off;
    const __amdgpu_buffer_rsrc_t rx = raw_rsrc(X + (int64_t)k0 * D, (uint32_t)BN * D * 2);
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = (j * NW + w) * 64 * 8;
      const uint32_t sj = J_INV ? j * J_STEP : 0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(Xs + blk), 16, off[J_INV ? 0 : j], sj, 0, 0);
    }
  }
  // issue() through dma16_asm
  template <bool IS_K>
  __device__ __forceinline__ void issue_asm(const bf16* X, bf16* Xs, int k0, int n_s, int w) const {
    const uint32_t* off = IS_K ? k_off : v_off;
    const int rows = min(BN, n_s - k0);
    const u32x4 rx = asm_rsrc(X + (int64_t)k0 * D, (uint32_t)rows * D * 2);
    const uint32_t lim = (uint32_t)rows * (2 * D);
    const uint32_t last = lim - 2 * D;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = (j * NW + w) * 64 * 8;
      if (rows == BN) {
        dma16_asm(Xs + blk, rx, off[J_INV ? 0 : j], J_INV ? j * J_STEP : 0u);
      } else {
        const uint32_t xj = J_INV ? off[0] + j * J_STEP : off[j];
        dma16_asm(Xs + blk, rx, xj < lim ? xj : last + (xj & (2 * D - 1)), 0u);
      }
    }
  }
};


// Byte offset, in a "V"-layout tile of D columns, of lane `lane`'s first
// transposing read for the 32-column block cb of an MFMA operand whose k
// index runs down the rows: lane 16G + 4a + b reads rows 16p + 8s + 4h + a
// (k chunk p, s = 0 for elements 0..3, s = 1 for 4..7) and columns
// 32cb + 16(G % 2) + 4b .. + 3. The row's swizzle depends on a only, so k
// chunk p and s add 32pD and 16D bytes.
template <int D>
__device__ __forceinline__ uint32_t tr_offset(int lane, int cb) {
  const int h = lane >> 5, G = lane >> 4, a = (lane >> 2) & 3, b = lane & 3;
  const int r0 = 4 * h + a;
  const int col = 32 * cb + 16 * (G & 1) + 4 * b;
  return 2 * (r0 * D + 8 * ((col >> 3) ^ swz_v<D>(r0)) + (col & 7));
}

// The 8-element operand fragment of k chunk p (16 rows) read transposed at
// lane offset `off` (tr_offset).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* tile, uint32_t off, int p) {
  const bf16x4 lo = lds_read_tr(lds_at(tile, off + 2 * 16 * p * D));
  const bf16x4 hi = lds_read_tr(lds_at(tile, off + 2 * (16 * p + 8) * D));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same transposing read on a "K"-layout tile (rows swizzled by swz_k, as
// read row-wise by the 16-byte operand loads), so one tile serves both kinds
// of operand. The row swizzle of row 16p + 8s + 4h + a depends on s but not
// on p, so a lane keeps two offsets per 32-column block: tr_offset_k(lane,
// cb, s), and fragment p reads offset s at + 32 p D bytes.
template <int D>
__device__ __forceinline__ uint32_t tr_offset_k(int lane, int cb, int s) {
  const int h = lane >> 5, G = lane >> 4, a = (lane >> 2) & 3, b = lane & 3;
  const int r = 8 * s + 4 * h + a;
  const int col = 32 * cb + 16 * (G & 1) + 4 * b;
  return 2 * (r * D + 8 * ((col >> 3) ^ swz_k<D>(r)) + (col & 7));
}
template <int D>
__device__ __forceinline__ bf16x8 tr_frag_k(const bf16* tile, uint32_t off0, uint32_t off1,
                                            int p) {
  const bf16x4 lo = lds_read_tr(lds_at(tile, off0 + 2 * 16 * p * D));
  const bf16x4 hi = lds_read_tr(lds_at(tile, off1 + 2 * 16 * p * D));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (DMA loads into LDS count, in issue order); LDS and export counters free.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Sum of x over aligned groups of G lanes (G = 2, 4, 8 or 16), every lane of a
// group getting the sum: DPP butterflies within a 16-lane row.
template <int G>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2..16 lanes");
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 decltype(ctrl)::value, 0xf, 0xf,
                                                                 false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});                        // quad_perm 1,0,3,2
  if constexpr (G >= 4) x += dpp(x, std::integral_constant<int, 0x4E>{});  // quad_perm 2,3,0,1
  if constexpr (G >= 8) x += dpp(x, std::integral_constant<int, 0x141>{}); // row_half_mirror
  if constexpr (G >= 16) x += dpp(x, std::integral_constant<int, 0x140>{});// row_mirror
  return x;
}

// Maximum and sum of x over the whole wave, returned to every lane: DPP
// butterflies within each 16-lane row, then the four rows combined through
// lanes 15, 31, 47 and 63 read with v_readlane.
__device__ __forceinline__ float wave_max(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 decltype(ctrl)::value, 0xf, 0xf,
                                                                 false));
  };
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0xB1>{}));
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0x4E>{}));
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0x141>{}));
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0x140>{}));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum<16>(x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace infini
