// Host-side check of the packed tile layouts (TileLayout in common.hpp), built and run by
// tests/test_tile_layout.py. Exit status 0 and "ok" on success.
//
// Checked against the operand definition of v_mfma_f32_32x32x16_bf16 (lane l supplies 8
// consecutive k of row l % 32 of A; k = 8 (l / 32) + [0, 8) within each 16-k step;
// accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4):
//  1. both layouts are bijections of the 64 x D tile;
//  2. K-type fragment (half, ks), lane 32 g + R, element u holds key 32 half + key_of_row(R),
//     column 16 ks + 8 g + u, and the score register r of lane half g then holds key
//     16 (r / 8) + 8 g + r % 8 of the half (so registers [8 ks, 8 ks + 8) are the PV k-step);
//  3. V-type fragment (half, et, ks), lane 32 g + l, element u holds key
//     32 half + 16 ks + 8 g + u, column 32 et + l (the PV A operand with that key order);
//  4. the chunk decoders name the first element of every 16-byte chunk.
#include <cstdio>
#include <vector>

#include "common.hpp"

using namespace pisa;

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      if (fails < 10) std::printf("fail: %s (line %d)\n", #c, __LINE__); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

template <class T, int D>
static void check() {
  using TL = TileLayout<T, D>;
  std::vector<int> seen_k(64 * D, 0), seen_v(64 * D, 0);
  for (int key = 0; key < 64; ++key)
    for (int c = 0; c < D; ++c) {
      ++seen_k[TL::k(key, c)];
      ++seen_v[TL::v(key, c)];
    }
  for (int x = 0; x < 64 * D; ++x) CHECK(seen_k[x] == 1 && seen_v[x] == 1);
  const int epc = 16 / int(sizeof(T));
  for (int x = 0; x < 64 * D / epc; ++x) {
    int key0 = -1, e = -1;
    TL::vchunk(x, key0, e);
    for (int u = 0; u < epc; ++u) CHECK(TL::v(key0 + u, e) == x * epc + u);
  }
  if constexpr (sizeof(T) == 2) {
    for (int half = 0; half < 2; ++half)
      for (int ks = 0; ks < D / 16; ++ks)
        for (int lane = 0; lane < 64; ++lane)
          for (int u = 0; u < 8; ++u) {
            const int g = lane >> 5, R = lane & 31;
            const int off = ((half * (D / 16) + ks) * 64 + lane) * 8 + u;
            CHECK(TL::k(32 * half + key_of_row(R), 16 * ks + 8 * g + u) == off);
          }
    for (int half = 0; half < 2; ++half)
      for (int et = 0; et < D / 32; ++et)
        for (int ks = 0; ks < 2; ++ks)
          for (int lane = 0; lane < 64; ++lane)
            for (int u = 0; u < 8; ++u) {
              const int g = lane >> 5, l = lane & 31;
              const int off = (((half * (D / 32) + et) * 2 + ks) * 64 + lane) * 8 + u;
              CHECK(TL::v(32 * half + 16 * ks + 8 * g + u, 32 * et + l) == off);
            }
    for (int x = 0; x < 64 * D / 8; ++x) {
      int key = -1, c0 = -1;
      TL::kchunk(x, key, c0);
      for (int u = 0; u < 8; ++u) CHECK(TL::k(key, c0 + u) == x * 8 + u);
    }
  }
}

int main() {
  for (int R = 0; R < 32; ++R) CHECK(row_of_key(key_of_row(R)) == R);
  for (int g = 0; g < 2; ++g)
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r / 4) + 4 * g + r % 4;           // accumulator row of register r
      CHECK(key_of_row(row) == 16 * (r / 8) + 8 * g + r % 8);
    }
  check<uint16_t, 64>();
  check<uint16_t, 128>();
  check<float, 64>();
  check<float, 128>();
  std::printf(fails ? "FAILED %d\n" : "ok\n", fails);
  return fails ? 1 : 0;
}
