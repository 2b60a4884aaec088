// Index arithmetic of the grouped LDS tile layout for head dimension 128
// (used through GrpTile128 and GrpCopy in common.hpp).  Plain constexpr
// integer functions, compiled for the GPU and, by the layout check under
// tests/, for the host.
//
// A 64-row (or any multiple of 16) tile of 128 bf16 per row.  Rows form
// groups of four, each group one direct-copy instruction's kilobyte
// (64 lanes x 16 bytes):
//   row k  -> group 4 (k >> 4) + (k & 3), slot (k >> 2) & 3;
//   groups -> GS = 1088 bytes apart (a 64-byte gap after each kilobyte);
//   16-byte chunk c (columns 8c .. 8c+7) of a row at slot a -> chunk
//   position c ^ a inside the row.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MATTN_HD __host__ __device__
#else
#define MATTN_HD
#endif

namespace mattn {
namespace grp {

constexpr int D = 128;
constexpr int ROW_BYTES = 2 * D;  // 256
constexpr int GS = 1088;          // bytes from one group to the next

MATTN_HD constexpr int group_of(int k) { return 4 * (k >> 4) + (k & 3); }
MATTN_HD constexpr int slot_of(int k) { return (k >> 2) & 3; }
// First tile row of group G (the row at slot 0).
MATTN_HD constexpr int group_row(int G) { return 16 * (G >> 2) + (G & 3); }
// Tile byte offset of chunk c of row k.
MATTN_HD constexpr int chunk_addr(int k, int c) {
  return group_of(k) * GS + ROW_BYTES * slot_of(k) + 16 * (c ^ slot_of(k));
}
// Byte offset, from the first row of its group, of the global chunk that
// lane L of a group's copy brings to tile offset (group base + 16 L):
// slot L >> 4, chunk position L & 15.
MATTN_HD constexpr unsigned copy_lane_off(int L) {
  return (unsigned)(4 * (L >> 4) * D + 8 * ((L & 15) ^ (L >> 4))) * 2u;
}
// Copy of a tile by CW waves (CW a multiple of 4): wave w takes groups
// w, w + CW, w + 2 CW, ...; in round r its lane L reads the global byte
// offset copy_off(w, L, r) from the tile's first row and writes 16 bytes at
// tile offset copy_dst(w, r) + 16 L.  Each round moves 4 CW rows, so the
// round term is a constant.
MATTN_HD constexpr unsigned copy_off(int CW, int w, int L, int r) {
  return copy_lane_off(L) + (unsigned)group_row(w) * ROW_BYTES + (unsigned)(r * 4 * CW * ROW_BYTES);
}
MATTN_HD constexpr int copy_dst(int CW, int w, int r) { return (w + r * CW) * GS; }
// Row operand (MFMA A: lane row l32 = lane & 31, columns 16 st + 8 g .. +7
// with g = lane >> 5) of tile rows row0 .. row0+31, row0 % 16 == 0:
// base for k-step parity e, and the full address.
MATTN_HD constexpr int row_base(int lane, int e) {
  return group_of(lane & 31) * GS + ROW_BYTES * slot_of(lane & 31) +
         16 * ((2 * e + (lane >> 5)) ^ slot_of(lane & 31));
}
MATTN_HD constexpr int row_addr(int lane, int row0, int st) {
  return (row0 >> 4) * 4 * GS + 64 * (st >> 1) + row_base(lane, st & 1);
}
// Transposed read (ds_read_b64_tr_b16) of tile rows row0 + 8h .. row0 + 8h + 7,
// columns 32 db .. 32 db + 31, row0 % 16 == 0: lane (j = lane >> 4,
// s = lane & 15) supplies the address of row row0 + 8h + 4 (j >> 1) + (s >> 2),
// columns 32 db + 16 (j & 1) + 4 (s & 3) .. +3.
MATTN_HD constexpr int trans_base(int lane, int h) {
  return ((lane & 15) >> 2) * GS + ROW_BYTES * (2 * h + (lane >> 5)) +
         16 * ((2 * ((lane >> 4) & 1) + ((lane >> 1) & 1)) ^ (2 * h + (lane >> 5))) +
         8 * (lane & 1);
}
MATTN_HD constexpr int trans_addr(int lane, int row0, int db, int h) {
  return (row0 >> 4) * 4 * GS + 64 * db + trans_base(lane, h);
}

}  // namespace grp

// Output staging (store_rows_bf16 in common.hpp): one wave's 32 rows of
// head dim d bf16 in LDS at row pitch 2d + 16 bytes.  Lane (l32 = lane & 31,
// g = lane >> 5) writes its 8 bytes of columns 32 db + 8 r + 4 g .. +3 of row
// l32; rows 16-31 keep the two 8-byte halves of each 16-byte chunk swapped.
namespace stage {
MATTN_HD constexpr int pitch(int d) { return 2 * d + 16; }
MATTN_HD constexpr int bytes(int d) { return 32 * pitch(d); }
MATTN_HD constexpr int write_off(int d, int lane, int db, int r) {
  return (lane & 31) * pitch(d) + (db * 32 + r * 8) * 2 + 8 * ((lane >> 5) ^ ((lane & 31) >> 4));
}
// Read-back: store instruction i, lane -> row and 16-byte chunk; rows of one
// instruction lie on one side of row 16 (swapped halves iff row >= 16).
MATTN_HD constexpr int read_row(int d, int i, int lane) { return i * (64 / (d / 8)) + lane / (d / 8); }
MATTN_HD constexpr int read_chunk(int d, int lane) { return lane % (d / 8); }
MATTN_HD constexpr int read_off(int d, int i, int lane) {
  return read_row(d, i, lane) * pitch(d) + 16 * read_chunk(d, lane);
}
MATTN_HD constexpr bool read_swapped(int d, int i) { return i * (64 / (d / 8)) >= 16; }
}  // namespace stage
}  // namespace mattn
