// Shared device helpers for the libmattn kernels (gfx950 / CDNA4).
//
// Matrix-core building block: v_mfma_f32_32x32x16_bf16, one wave64, fp32
// accumulate.  Operand layouts (lane l, l32 = l % 32, g = l / 32):
//   A (32 x 16): lane holds row l32, k = 8g .. 8g+7   (8 bf16, 16 bytes)
//   B (16 x 32): lane holds col l32, k = 8g .. 8g+7
//   C (32 x 32): lane holds col l32, rows ((i/4)*8 + 4g + i%4), i = 0..15
// A C tile can feed the next MFMA as its B operand directly (lane keeps its
// column): register i = 8t + e of the C tile becomes k-slot 8g + e of k-step
// t.  The row it carries is 16t + swz(8g + e), where swz swaps bits 2 and 3
// of a 4-bit index.  The other operand of that MFMA is therefore read from
// LDS in the same permuted order (ld_trans_operand below); since a
// contraction is a sum, the order is free.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grp_layout.hpp"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define MATTN_INF __builtin_huge_valf()
#define MATTN_LOG2E 1.4426950408889634f
#define MATTN_LN2 0.6931471805599453f

namespace mattn {

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the C tile held by register i of lane group g.
__device__ __forceinline__ constexpr int crow(int i, int g) {
  return (i >> 2) * 8 + g * 4 + (i & 3);
}

// LDS tile pitches (bf16 elements).  A [rows x D] tile is stored row-major
// with a padded pitch chosen for the way it is read (64 four-byte banks, 256
// bytes):
//   * row operands: 16 lanes read 16 bytes from 16 consecutive rows; pitch
//     304 B (D = 128) / 208 B (D = 64) puts them in 16 distinct bank quads;
//   * transposed operands: 32 lanes read 64 bytes from each of 4 consecutive
//     rows; pitch 320 B (D = 128) / 192 B (D = 64) puts the 4 rows in
//     disjoint 64-byte bank segments.
// No single pitch serves both.  Measured on MI355X: 197 (rows, 304 B) and 182
// (transposed, 320 B) bytes per clock per CU, against 62 and 116 with the
// pitches swapped.  A tile that is read both ways is stored once, in the
// swizzled layout of SwzTile below.
template <int D>
struct RowPitch {
  static constexpr int value = D == 128 ? 152 : 104;
};
template <int D>
struct TrPitch {
  static constexpr int value = D == 128 ? 160 : 96;
};

// A operand of mfma32 read straight from a row-major tile in LDS: lane row
// l32 = tile row row0 + l32, k-slots 8g..8g+7 = columns col0 + 8g ...
__device__ __forceinline__ bf16x8 ld_row_operand(const bf16* tile, int pitch, int row0, int col0,
                                                 int lane) {
  return *reinterpret_cast<const bf16x8*>(&tile[(row0 + (lane & 31)) * pitch + col0 + 8 * (lane >> 5)]);
}

// A operand of mfma32 holding the TRANSPOSE of a row-major tile in LDS:
// operand row r (lane row l32) is tile column col0 + r, and k-slot 8g + e of
// the k-step is tile row row0 + swz(8g + e), the order in which a C tile fed
// as the B operand carries its rows.  Built from two ds_read_b64_tr_b16: in
// each 16-lane group that instruction hands lane i element (i % 4) of the
// 8-byte chunk read by source lane 4e + i/4, so source lane s of group j
// reads tile row row0 + 8h + 4(j/2) + s/4 at columns col0 + 16(j%2) + 4(s%4)
// .. +3.  `pitch` must be a multiple of 4.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// One ds_read_b64_tr_b16.  The compiler tracks direct global->LDS copies in
// flight per LDS object (the alias scopes it gives each __shared__ variable),
// so a read of one buffer only waits for copies into that same buffer; a
// kernel that keeps its double buffers in separate __shared__ variables can
// read one while copies into the other are still in flight.
__device__ __forceinline__ bf16x4_t ds_read_tr(const lds_bf16x4* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p));
}

__device__ __forceinline__ bf16x8 ld_trans_operand(const bf16* tile, int pitch, int row0,
                                                   int col0, int lane) {
  const int j = lane >> 4, s = lane & 15;
  const bf16* p = tile + (row0 + 4 * (j >> 1) + (s >> 2)) * pitch + col0 + 16 * (j & 1) + 4 * (s & 3);
  const bf16x4_t lo = ds_read_tr((const lds_bf16x4*)(p));
  const bf16x4_t hi = ds_read_tr((const lds_bf16x4*)(p + 8 * pitch));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ld_trans_operand with the lane-dependent part of the address computed once.
// The compiler attaches an LDS object's alias scope only to accesses whose
// address it can trace back to that object through a few address steps; an
// address built from several separately combined lane terms can lose it, and
// the read then waits for every direct copy in flight.  Here the lane term is
// one opaque value, so each read's address is the tile base + that value + a
// compile-time constant.
struct TransReader {
  int off;  // element offset of this lane's first chunk for row0 = col0 = 0
  __device__ __forceinline__ void init(int pitch, int lane) {
    const int j = lane >> 4, s = lane & 15;
    off = (4 * (j >> 1) + (s >> 2)) * pitch + 16 * (j & 1) + 4 * (s & 3);
    asm volatile("" : "+v"(off));
  }
  __device__ __forceinline__ bf16x8 operator()(const bf16* tile, int pitch, int row0,
                                               int col0) const {
    const bf16* p = tile + off;
    const bf16x4_t lo = ds_read_tr((const lds_bf16x4*)(p + row0 * pitch + col0));
    const bf16x4_t hi = ds_read_tr((const lds_bf16x4*)(p + (row0 + 8) * pitch + col0));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Layout of a [rows x D] bf16 tile in LDS that is read both as row operands
// and transposed: pitch TrPitch<D>, and the 16-byte chunk c of row r held at
// chunk position c ^ ((r >> 2) & 3).  At that pitch the four rows of a
// transposed read already fall in disjoint 64-byte bank segments, and the XOR
// (which only permutes chunks inside aligned 64-byte blocks) leaves that
// intact, while it moves the sixteen rows of a row read, which the pitch
// alone maps onto four segments, onto sixteen distinct 16-byte bank groups.
// Because the XOR touches only the low two bits of the chunk index, a lane's
// address for any k-step or d-block is one of two per-lane bases plus a
// compile-time offset.  Reads start at rows that are multiples of 16.
template <int D>
struct SwzTile {
  static constexpr int P = TrPitch<D>::value;
  int rbase[2];  // row operand, k-step parity b: row l32, chunk (2b + g) ^ F(l32)
  int tbase[2];  // transposed operand, rows 0..7 (h = 0) and 8..15 (h = 1) of a 16-row step
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int b = 0; b < 2; ++b) rbase[b] = l32 * P + 8 * ((2 * b + g) ^ ((l32 >> 2) & 3));
    const int j = lane >> 4, s = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 4 * (j >> 1) + (s >> 2) + 8 * h;
      tbase[h] = r * P + 8 * ((2 * (j & 1) + ((s >> 1) & 1)) ^ ((r >> 2) & 3)) + 4 * (s & 1);
    }
    // Opaque to the optimizer, so that every read's address stays the tile
    // base + one lane value + a constant (see TransReader).
    asm volatile("" : "+v"(rbase[0]), "+v"(rbase[1]), "+v"(tbase[0]), "+v"(tbase[1]));
  }
  // Element offset of the chunk that holds columns 8*chunk .. 8*chunk+7 of row `row`.
  static __device__ __forceinline__ int store_off(int row, int chunk) {
    return row * P + 8 * (chunk ^ ((row >> 2) & 3));
  }
  // ld_row_operand of this layout: rows row0 .. row0+31, columns 16st .. 16st+15.
  __device__ __forceinline__ bf16x8 row(const bf16* tile, int row0, int st) const {
    return *reinterpret_cast<const bf16x8*>(tile + row0 * P + 32 * (st >> 1) + rbase[st & 1]);
  }
  // ld_trans_operand of this layout: operand rows = tile columns 32db .. 32db+31,
  // k-slots = tile rows row0 + swz(8g + e), as there.
  __device__ __forceinline__ bf16x8 trans(const bf16* tile, int row0, int db) const {
    const bf16* p = tile + row0 * P + 32 * db;
    const bf16x4_t lo = ds_read_tr((const lds_bf16x4*)(p + tbase[0]));
    const bf16x4_t hi = ds_read_tr((const lds_bf16x4*)(p + tbase[1]));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// The grouped layout of a [rows x 128] bf16 tile in LDS (rows a multiple of
// 16; index arithmetic in grp_layout.hpp), read both as row operands and
// transposed and filled by direct copies that write data only, no padding.
// Rows form groups of four, each one copy instruction's kilobyte, and groups
// sit 1088 bytes apart, so the four groups of rows k, k+1, k+2, k+3 start in
// four different 64-byte bank segments:
//  * a transposed read's four rows of one lane group are those four rows, one
//    per segment, and the chunk XOR (by slot) keeps the two lane groups of a
//    pass apart;
//  * a row read's sixteen rows fill the four slots of four groups: the group
//    picks the segment and the XOR the 16-byte bank group within it.
// Both reads are then free of bank conflicts, and a lane's address for any
// k-step or d-block is one of two per-lane bases plus a compile-time offset.
// Reads start at rows that are multiples of 16.
struct GrpTile128 {
  static constexpr int D = grp::D;
  static constexpr int GS = grp::GS;
  static constexpr int bytes(int rows) { return rows / 4 * GS; }
  int rbase[2];  // row operand, k-step parity e (bytes)
  int tbase[2];  // transposed operand, rows 0..7 (h = 0) and 8..15 (h = 1) of a 16-row step
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int e = 0; e < 2; ++e) rbase[e] = grp::row_base(lane, e);
#pragma unroll
    for (int h = 0; h < 2; ++h) tbase[h] = grp::trans_base(lane, h);
    asm volatile("" : "+v"(rbase[0]), "+v"(rbase[1]), "+v"(tbase[0]), "+v"(tbase[1]));
  }
  // A operand rows row0 .. row0+31, columns 16st .. 16st+15 (as ld_row_operand).
  __device__ __forceinline__ bf16x8 row(const bf16* tile, int row0, int st) const {
    const char* p = reinterpret_cast<const char*>(tile) + (row0 >> 4) * 4 * GS + 64 * (st >> 1);
    return *reinterpret_cast<const bf16x8*>(p + rbase[st & 1]);
  }
  // A operand rows = tile columns 32db .. 32db+31, k-slots = tile rows
  // row0 .. row0+15 (as TransReader).
  __device__ __forceinline__ bf16x8 trans(const bf16* tile, int row0, int db) const {
    const char* p = reinterpret_cast<const char*>(tile) + (row0 >> 4) * 4 * GS + 64 * db;
    const bf16x4_t lo = ds_read_tr((const lds_bf16x4*)(p + tbase[0]));
    const bf16x4_t hi = ds_read_tr((const lds_bf16x4*)(p + tbase[1]));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.0f;
  return z;
}

// Range-checked raw buffer access.  The descriptor covers `nbytes` bytes from
// a wave-uniform base; a load whose offset falls outside returns zero without
// touching memory, so tile loads over ragged tails need no branches.
// Descriptor word 3 selects 32-bit data format, the plain gfx9 raw-buffer
// setting.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Buf(const void* base, uint32_t nbytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                            0x00020000)) {}
  __device__ __forceinline__ uint4 ld16(uint32_t off) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ uint32_t ld4(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ float ldf(uint32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
};

// Workgroup barrier for loops whose LDS traffic between barriers is reads
// plus direct copies that each wave has already waited for (s_waitcnt
// vmcnt).  __syncthreads() adds a release fence, which waits for every
// outstanding vector memory operation, including direct copies issued for
// later tiles; this barrier leaves those in flight.  The empty asm statements
// keep the compiler from moving memory accesses across it.  Not for use after
// ds_write: those need the fence (or an explicit lgkmcnt wait) first.
__device__ __forceinline__ void barrier_keep_copies() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global -> LDS copy of 16 bytes per lane: lane L's bytes land at
// lds_base + 16 L (lds_base wave-uniform).  Offsets outside the descriptor's
// range write zeros.  Completion is tracked by vmcnt, like other vector
// memory loads.
__device__ __forceinline__ void ld16_to_lds(const Buf& b, uint32_t off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           off, 0, 0, 0);
}
// The same with 4 bytes per lane: lane L's word lands at lds_base + 4 L.
__device__ __forceinline__ void ld4_to_lds(const Buf& b, uint32_t off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (__attribute__((address_space(3))) void*)lds_base, 4,
                                           off, 0, 0, 0);
}

// A tile of `ROWS` rows x D bf16 with row pitch PITCH (elements), filled by
// ld16_to_lds.  The tile's LDS bytes are split into 16-byte slots, slot q =
// row * (PITCH / 8) + chunk; the workgroup's NT threads cover the slots in
// rounds of NT, so each wave writes one contiguous kilobyte per round.  A
// slot in a row's padding gets an out-of-range offset and is written as
// zeros.  The per-thread global offsets depend only on the thread, so they
// are computed once; per tile only the descriptor base moves.
template <int D, int ROWS, int PITCH, int NT>
struct DirectTile {
  static constexpr int SLOTS_PER_ROW = PITCH / 8;
  static constexpr int SLOTS = ROWS * SLOTS_PER_ROW;
  static constexpr int ROUNDS = (SLOTS + NT - 1) / NT;
  // LDS elements to allocate: whole waves of slots, so a wave that straddles
  // the tile's end writes its surplus slots (as zeros) into padding.
  static constexpr int LDS_ELEMS = (SLOTS + 63) / 64 * 64 * 8;
  static_assert(PITCH % 8 == 0 && PITCH >= D, "pitch");
  uint32_t off[ROUNDS];
  int w0;  // first slot of this wave in round 0; wave-uniform, kept in a scalar register
  __device__ __forceinline__ void init(int tid) {
    w0 = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int q = r * NT + tid;
      const int row = q / SLOTS_PER_ROW, c = q - row * SLOTS_PER_ROW;
      off[r] = (q < SLOTS && c < D / 8) ? (uint32_t)(row * D + c * 8) * 2 : 0x80000000u;
    }
  }
  // Copy rows [0, ROWS) of `src` (a descriptor whose base is the tile's first
  // row) into `lds` (the tile, PITCH-padded, LDS_ELEMS long).  Waves whose
  // slots all lie past the tile's end skip the round.
  __device__ __forceinline__ void load(const Buf& src, bf16* lds, int tid) const {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int q0 = r * NT + w0;  // first slot of this wave in round r
      if (SLOTS % NT == 0 || q0 < SLOTS)
        ld16_to_lds(src, off[r], lds + q0 * 8);
    }
  }
};

// Direct copy of a ROWS-row tile into the GrpTile128 layout by CW waves:
// wave w takes groups w, w + CW, w + 2 CW, ...  Every lane's global offset
// is one register (the group's first row is a per-wave and per-round
// constant: with CW a multiple of 4 each round moves 4 CW rows), and each
// copy instruction writes one whole group, so no padding is written.
template <int ROWS, int CW>
struct GrpCopy {
  static constexpr int GROUPS = ROWS / 4;
  static constexpr int ROUNDS = GROUPS / CW;
  static_assert(ROWS % 16 == 0 && CW % 4 == 0 && GROUPS % CW == 0, "whole rounds");
  uint32_t voff;  // bytes from the tile's first row, round 0
  int lds0;       // byte offset of this wave's round-0 group (wave-uniform)
  __device__ __forceinline__ void init(int w, int lane) {
    voff = grp::copy_off(CW, w, lane, 0);
    lds0 = grp::copy_dst(CW, w, 0);
  }
  // src: a descriptor whose base is the tile's first row and whose range ends
  // at the last valid row, so rows past it land as zeros.
  __device__ __forceinline__ void load(const Buf& src, void* tile) const {
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r)
      ld16_to_lds(src, voff + (grp::copy_off(CW, 0, 0, r) - grp::copy_off(CW, 0, 0, 0)),
                  reinterpret_cast<char*>(tile) + lds0 + (grp::copy_dst(CW, 0, r) - grp::copy_dst(CW, 0, 0)));
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16 x = (bf16)a, y = (bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Two floats as fp16, rounded to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}

// Bytes of LDS that store_rows_bf16 stages one wave's 32 rows in.
template <int D>
constexpr int stage_rows_bytes() { return stage::bytes(D); }

// Store of a wave's 32 output rows held in the MFMA C layout (lane column
// l32 = row; register i of block db = column 32db + 8(i/4) + 4g + i%4, with
// g = lane >> 5), scaled by mul and rounded to bf16.  Written directly, every
// store instruction would touch 32 rows at 16 bytes each; instead the rows
// go through wave-private LDS (stg: stage_rows_bytes<D>() bytes; layout and
// offsets in grp_layout.hpp, namespace stage) and come back so that each
// store instruction writes whole consecutive rows, 64 lanes x 16 bytes.
// Rows at or past rows_valid (counted from the first) are not written.  The
// LDS writes and reads are the same wave's, in program order, so no barrier
// is involved.  Rows 16-31 are staged with the 8-byte halves of each chunk
// swapped (a half-wave's 8-byte writes to rows r and r+16 would otherwise
// share banks); their read-back swaps them again.
template <int D>
__device__ __forceinline__ void store_rows_bf16(const f32x16 (&acc)[D / 32], float mul, char* stg,
                                                bf16* out, int rows_valid, int lane) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint2 w;
      w.x = pack_bf16x2(acc[db][4 * r] * mul, acc[db][4 * r + 1] * mul);
      w.y = pack_bf16x2(acc[db][4 * r + 2] * mul, acc[db][4 * r + 3] * mul);
      *reinterpret_cast<uint2*>(stg + stage::write_off(D, lane, db, r)) = w;
    }
  static_assert(16 % (64 / (D / 8)) == 0, "an instruction's rows lie on one side of row 16");
#pragma unroll
  for (int i = 0; i < 32 / (64 / (D / 8)); ++i) {
    const int row = stage::read_row(D, i, lane), ch = stage::read_chunk(D, lane);
    uint4 v = *reinterpret_cast<const uint4*>(stg + stage::read_off(D, i, lane));
    if (stage::read_swapped(D, i)) v = make_uint4(v.z, v.w, v.x, v.y);
    if (row < rows_valid) *reinterpret_cast<uint4*>(out + (size_t)row * D + ch * 8) = v;
  }
}

// Workgroup -> (head, query tile) order, assuming round-robin dispatch of
// consecutive workgroup ids over the 8 XCDs (id % 8 = XCD), each with its own
// L2.  Non-causal: head-major, remapped so that each XCD walks a contiguous
// run of tiles (tiles of one head share K/V, which then stays in that XCD's
// L2).  Causal: longest query tiles first across the whole grid, and inside
// each tile level each XCD takes a contiguous run of heads, the same run at
// every level, so grouped query heads and their K/V stay on one XCD.
__device__ __forceinline__ void tile_of_block(int p, int nbh, int n_qt, bool causal, int& bh,
                                              int& qt) {
  if (causal) {
    const int level = p / nbh, r = p - level * nbh;
    bh = ((nbh & 7) == 0) ? (r & 7) * (nbh >> 3) + (r >> 3) : r;
    qt = n_qt - 1 - level;
  } else {
    const int N = nbh * n_qt;
    const int L = ((N & 7) == 0) ? (p & 7) * (N >> 3) + (p >> 3) : p;
    bh = L / n_qt;
    qt = L - bh * n_qt;
  }
}

__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace mattn
