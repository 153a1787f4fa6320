// Host codec under AddressSanitizer and UndefinedBehaviorSanitizer: every
// buffer is allocated at exactly the size the C ABI documents, so a read or
// write one byte past it is reported.  Exercises moe_pack, moe_unpack,
// moe_tile_container and moe_untile_container on both containers: round
// trips, every value of every byte position of a block, and the error paths
// (which must leave the destination untouched).  Prints "ok" and returns 0 when
// every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "moe_ternary.h"

static int g_bad = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_bad;                                                        \
    }                                                                 \
  } while (0)

// A heap buffer of exactly n bytes (n may be 0): an access past it is an error.
struct Buf {
  uint8_t* p;
  int64_t n;
  explicit Buf(int64_t bytes) : p(new uint8_t[bytes > 0 ? bytes : 1]), n(bytes) {}
  ~Buf() { delete[] p; }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

static void round_trip(int fmt, int64_t n, std::mt19937& rng) {
  std::vector<int8_t> t(n);
  std::vector<uint16_t> s(n / 128);
  std::uniform_int_distribution<int> tri(-1, 1);
  std::uniform_int_distribution<int> bits(0, 0xFFFF);
  for (auto& v : t) v = (int8_t)tri(rng);
  for (auto& v : s) {
    do v = (uint16_t)bits(rng);
    while ((v & 0x7C00) == 0x7C00);  // finite scales only
  }
  const int64_t nb = moe_packed_bytes(fmt, n);
  CHECK(nb == n / 128 * moe_block_bytes(fmt));
  Buf packed(nb);
  CHECK(moe_pack(fmt, t.data(), s.data(), n, packed.p, packed.n) == MOE_OK);
  Buf t2(n), s2(2 * (n / 128));
  CHECK(moe_unpack(fmt, packed.p, packed.n, (int8_t*)t2.p, (uint16_t*)s2.p, n) == MOE_OK);
  CHECK(n == 0 || std::memcmp(t.data(), t2.p, (size_t)n) == 0);
  CHECK(n == 0 || std::memcmp(s.data(), s2.p, (size_t)(2 * (n / 128))) == 0);
  // one byte short: refused, nothing written
  if (nb > 0) {
    Buf shortb(nb - 1);
    std::memset(shortb.p, 0x5A, (size_t)shortb.n);
    CHECK(moe_pack(fmt, t.data(), s.data(), n, shortb.p, shortb.n) == MOE_E_SPACE);
    bool untouched = true;
    for (int64_t i = 0; i < shortb.n; ++i) untouched &= shortb.p[i] == 0x5A;
    CHECK(untouched);
    CHECK(moe_unpack(fmt, shortb.p, shortb.n, (int8_t*)t2.p, (uint16_t*)s2.p, n) == MOE_E_SPACE);
  }
}

// Every value of every byte position of one block, the others valid zeros.
static void every_byte(int fmt) {
  const int bb = (int)moe_block_bytes(fmt);
  Buf blk(bb), t(128), s(2);
  for (int pos = 0; pos < bb; ++pos) {
    for (int v = 0; v < 256; ++v) {
      std::memset(blk.p, 0, (size_t)bb);
      blk.p[pos] = (uint8_t)v;
      const int32_t rc = moe_unpack(fmt, blk.p, blk.n, (int8_t*)t.p, (uint16_t*)s.p, 128);
      bool valid;
      if (fmt == MOE_PQ2_0) {
        valid = pos >= 32 ? (((pos == 33 ? v << 8 : v) & 0x7C00) != 0x7C00)
                          : !(((v & 3) == 2) || (((v >> 2) & 3) == 2) || (((v >> 4) & 3) == 2) || ((v >> 6) == 2));
      } else {
        valid = pos < 24 ? v < 243 : pos < 26 ? v < 81 : (((pos == 27 ? v << 8 : v) & 0x7C00) != 0x7C00);
      }
      CHECK(valid ? rc == MOE_OK : rc != MOE_OK);
      if (!valid) CHECK(std::strlen(moe_last_error()) > 0);
    }
  }
}

static void tiling(int fmt, int64_t rows, int64_t cols, std::mt19937& rng) {
  const int64_t bytes = rows * cols / 128 * moe_block_bytes(fmt);
  Buf a(bytes), b(bytes), c(bytes);
  for (int64_t i = 0; i < bytes; ++i) a.p[i] = (uint8_t)rng();
  CHECK(moe_tile_container(fmt, a.p, rows, cols, b.p, b.n) == MOE_OK);
  CHECK(moe_untile_container(fmt, b.p, rows, cols, c.p, c.n) == MOE_OK);
  CHECK(bytes == 0 || std::memcmp(a.p, c.p, (size_t)bytes) == 0);
  if (bytes > 0) {
    Buf shortb(bytes - 1);
    CHECK(moe_tile_container(fmt, a.p, rows, cols, shortb.p, shortb.n) == MOE_E_SPACE);
    CHECK(moe_tile_container(fmt, a.p, rows, cols, a.p, a.n) == MOE_E_ARG);  // overlap
  }
  CHECK(moe_tile_container(fmt, a.p, rows + 1, cols, b.p, b.n) == MOE_E_SHAPE);
}

int main() {
  std::mt19937 rng(12345);
  for (int fmt : {MOE_PQ2_0, MOE_PTQ1_0}) {
    for (int64_t n : {0ll, 128ll, 256ll, 128ll * 37, 128ll * 1031}) round_trip(fmt, n, rng);
    every_byte(fmt);
    for (auto rc : {std::pair<int64_t, int64_t>{16, 128}, {32, 384}, {48, 1152}, {0, 128}, {16, 0}})
      tiling(fmt, rc.first, rc.second, rng);
  }
  // argument errors
  int8_t t[128] = {0};
  uint16_t s[1] = {0x3C00};
  uint8_t out[34];
  CHECK(moe_pack(99, t, s, 128, out, 34) == MOE_E_FORMAT);
  CHECK(moe_pack(MOE_PQ2_0, t, s, 100, out, 34) == MOE_E_SHAPE);
  CHECK(moe_pack(MOE_PQ2_0, nullptr, s, 128, out, 34) == MOE_E_ARG);
  t[5] = 2;
  CHECK(moe_pack(MOE_PQ2_0, t, s, 128, out, 34) == MOE_E_ARG);
  t[5] = 0;
  s[0] = 0x7C00;
  CHECK(moe_pack(MOE_PTQ1_0, t, s, 128, out, 34) == MOE_E_NONFINITE);
  CHECK(moe_packed_bytes(MOE_PQ2_0, -128) == -1 && moe_block_bytes(7) == -1);
  if (g_bad) {
    std::fprintf(stderr, "%d checks failed\n", g_bad);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
