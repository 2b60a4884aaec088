// Host check of the LDS layouts in grp_layout.hpp.  Grouped tile: the direct
// copies place every element of a 64 x 128 bf16 tile exactly once, the row
// and transposed operand addresses find the elements the MFMA operands need,
// and neither read pattern has bank conflicts (64 banks of 4 bytes; a row
// read serves 16 lanes x 16 bytes per pass, a transposed read 32 lanes x
// 8 bytes).  Output staging: placement, read-back and conflict-free writes.
// Prints "ok" and exits 0 on success.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "grp_layout.hpp"

using namespace mattn::grp;

static int fails = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      if (fails < 10) std::printf(__VA_ARGS__), std::printf("\n"); \
      ++fails;                                          \
    }                                                   \
  } while (0)

int main() {
  const int ROWS = 64, BYTES = ROWS / 4 * GS;
  // tile byte -> element index (row * D + col) of the bf16 it holds (-1: none)
  std::vector<int> at(BYTES, -1);
  for (int CW : {4, 8}) {
    std::fill(at.begin(), at.end(), -1);
    for (int w = 0; w < CW; ++w)
      for (int r = 0; r < ROWS / 4 / CW; ++r)
        for (int L = 0; L < 64; ++L) {
          const unsigned g = copy_off(CW, w, L, r);   // global byte offset from row 0
          const int dst = copy_dst(CW, w, r) + 16 * L;
          CHECK(g % 16 == 0 && g + 16 <= (unsigned)(ROWS * D * 2), "copy source out of tile");
          CHECK(dst >= 0 && dst + 16 <= BYTES, "copy destination out of tile");
          for (int e = 0; e < 8; ++e) {
            CHECK(at[dst + 2 * e] == -1, "tile byte written twice");
            at[dst + 2 * e] = (int)(g / 2) + e;
          }
        }
    int placed = 0;
    for (int x : at) placed += x >= 0;
    CHECK(placed == ROWS * D, "elements placed: %d", placed);
    for (int k = 0; k < ROWS; ++k)
      for (int c = 0; c < D / 8; ++c) CHECK(at[chunk_addr(k, c)] == k * D + 8 * c, "chunk_addr %d %d", k, c);
  }
  auto bank_worst = [](const std::vector<int>& addr, int lanes_per_pass, int bytes) {
    int worst = 0;
    for (size_t p0 = 0; p0 < addr.size(); p0 += lanes_per_pass) {
      std::map<int, int> cnt;
      for (int l = 0; l < lanes_per_pass; ++l)
        for (int b = 0; b < bytes / 4; ++b) worst = std::max(worst, ++cnt[(addr[p0 + l] / 4 + b) % 64]);
    }
    return worst;
  };
  // Row operand: lane (l32, g) needs row row0 + l32, columns 16 st + 8 g .. +7.
  for (int row0 = 0; row0 + 32 <= ROWS; row0 += 16)
    for (int st = 0; st < D / 16; ++st) {
      std::vector<int> addr(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int l32 = lane & 31, g = lane >> 5;
        addr[lane] = row_addr(lane, row0, st);
        for (int e = 0; e < 8; ++e)
          CHECK(at[addr[lane] + 2 * e] == (row0 + l32) * D + 16 * st + 8 * g + e, "row read %d %d %d", row0, st, lane);
      }
      CHECK(bank_worst(addr, 16, 16) == 1, "row read bank conflict row0=%d st=%d", row0, st);
    }
  // Transposed read: lane (j, s) supplies row row0 + 8h + 4 (j >> 1) + (s >> 2),
  // columns 32 db + 16 (j & 1) + 4 (s & 3) .. +3.
  for (int row0 = 0; row0 + 16 <= ROWS; row0 += 16)
    for (int db = 0; db < D / 32; ++db)
      for (int h = 0; h < 2; ++h) {
        std::vector<int> addr(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int j = lane >> 4, s = lane & 15;
          const int r = row0 + 8 * h + 4 * (j >> 1) + (s >> 2);
          const int col = 32 * db + 16 * (j & 1) + 4 * (s & 3);
          addr[lane] = trans_addr(lane, row0, db, h);
          for (int e = 0; e < 4; ++e)
            CHECK(at[addr[lane] + 2 * e] == r * D + col + e, "transposed read %d %d %d %d", row0, db, h, lane);
        }
        CHECK(bank_worst(addr, 32, 8) == 1, "transposed read bank conflict row0=%d db=%d h=%d", row0, db, h);
      }
  // Output staging: every (row, column) of a wave's 32 rows written once,
  // read back into the right place, half-wave 8-byte writes conflict free.
  for (int d : {64, 128}) {
    std::vector<int> st(mattn::stage::bytes(d), -1);
    for (int db = 0; db < d / 32; ++db)
      for (int r = 0; r < 4; ++r) {
        std::vector<int> addr(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int a = mattn::stage::write_off(d, lane, db, r);
          addr[lane] = a;
          CHECK(a >= 0 && a + 8 <= mattn::stage::bytes(d) && a % 8 == 0, "staging write out of range");
          for (int e = 0; e < 4; ++e) {
            CHECK(st[a + 2 * e] == -1, "staging byte written twice");
            st[a + 2 * e] = (lane & 31) * d + db * 32 + r * 8 + 4 * (lane >> 5) + e;
          }
        }
        CHECK(bank_worst(addr, 32, 8) == 1, "staging write bank conflict d=%d db=%d r=%d", d, db, r);
      }
    for (int i = 0; i < 32 / (64 / (d / 8)); ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const int a = mattn::stage::read_off(d, i, lane);
        CHECK(a % 16 == 0, "staging read misaligned");
        const int row = mattn::stage::read_row(d, i, lane), ch = mattn::stage::read_chunk(d, lane);
        for (int e = 0; e < 8; ++e) {
          const int src = mattn::stage::read_swapped(d, i) ? (e + 4) % 8 : e;
          CHECK(st[a + 2 * src] == row * d + 8 * ch + e, "staging read-back d=%d i=%d lane=%d", d, i, lane);
        }
      }
  }
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
