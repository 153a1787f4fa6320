// Host side of the container codec: pack, validate-and-unpack, the block
// reorder between moe_pack's row-major order and the expert kernels'
// tile-major order, and the error state of the C ABI.  Plain C++ (no device
// code), so it also builds with a host compiler alone, as the sanitizer test
// does.  Container layouts: Scion-35B-A3B card, "Weight Representation"
// (PQ2_0) and Scion-FlashNext card, "Weight Representation" (PTQ1_0); see
// include/moe_ternary.h.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "host_error.h"
#include "moe_ternary.h"

namespace moe {

namespace {
thread_local std::string g_err;

bool finite_f16(uint16_t h) { return (h & 0x7C00u) != 0x7C00u; }
}  // namespace

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t ok() {
  g_err.clear();
  return MOE_OK;
}

bool known_fmt(int32_t fmt) { return fmt == MOE_PQ2_0 || fmt == MOE_PTQ1_0; }

int32_t bad_fmt(int32_t fmt) {
  return fail(MOE_E_FORMAT, "unknown container id %d; valid ids are 142 (PQ2_0) and 143 (PTQ1_0)",
              (int)fmt);
}

}  // namespace moe

using moe::bad_fmt;
using moe::fail;
using moe::finite_f16;
using moe::known_fmt;
using moe::ok;

extern "C" {

const char* moe_last_error(void) { return moe::g_err.c_str(); }

int64_t moe_block_bytes(int32_t fmt) {
  if (fmt == MOE_PQ2_0) return 34;
  if (fmt == MOE_PTQ1_0) return 28;
  return -1;
}

int64_t moe_packed_bytes(int32_t fmt, int64_t n) {
  if (!known_fmt(fmt) || n < 0 || n % 128) return -1;
  return n / 128 * moe_block_bytes(fmt);
}

int32_t moe_pack(int32_t fmt, const int8_t* trits, const uint16_t* scales, int64_t n, uint8_t* dst,
                 int64_t dst_bytes) {
  try {
    if (!known_fmt(fmt)) return bad_fmt(fmt);
    if (n < 0 || n % 128) return fail(MOE_E_SHAPE, "weight count %lld is not a multiple of 128", (long long)n);
    if (n > 0 && (!trits || !scales || !dst)) return fail(MOE_E_ARG, "NULL pointer");
    const int64_t need = moe_packed_bytes(fmt, n);
    if (dst_bytes < need)
      return fail(MOE_E_SPACE, "dst holds %lld bytes, %lld needed", (long long)dst_bytes, (long long)need);
    const int64_t nb = n / 128;
    for (int64_t b = 0; b < nb; ++b)
      if (!finite_f16(scales[b])) return fail(MOE_E_NONFINITE, "non-finite fp16 scale in group %lld", (long long)b);
    for (int64_t i = 0; i < n; ++i)
      if (trits[i] < -1 || trits[i] > 1)
        return fail(MOE_E_ARG, "weight %lld is %d, not in {-1, 0, +1}", (long long)i, (int)trits[i]);
    if (fmt == MOE_PQ2_0) {
      for (int64_t b = 0; b < nb; ++b) {
        const int8_t* t = trits + b * 128;
        uint8_t* o = dst + b * 34;
        for (int j = 0; j < 32; ++j) {
          uint32_t v = 0;
          for (int i = 0; i < 4; ++i) v |= (uint32_t)(t[4 * j + i] & 3) << (2 * i);  // 0->00, 1->01, -1->11
          o[j] = (uint8_t)v;
        }
        o[32] = (uint8_t)(scales[b] & 0xFF);
        o[33] = (uint8_t)(scales[b] >> 8);
      }
    } else {
      for (int64_t b = 0; b < nb; ++b) {
        const int8_t* t = trits + b * 128;
        uint8_t* o = dst + b * 28;
        auto digit = [](int8_t v) { return v < 0 ? 2u : (uint32_t)v; };
        for (int j = 0; j < 24; ++j) {
          uint32_t v = 0, p = 1;
          for (int i = 0; i < 5; ++i, p *= 3) v += digit(t[5 * j + i]) * p;
          o[j] = (uint8_t)v;
        }
        for (int m = 0; m < 2; ++m) {
          uint32_t v = 0, p = 1;
          for (int i = 0; i < 4; ++i, p *= 3) v += digit(t[120 + 4 * m + i]) * p;
          o[24 + m] = (uint8_t)v;
        }
        o[26] = (uint8_t)(scales[b] & 0xFF);
        o[27] = (uint8_t)(scales[b] >> 8);
      }
    }
    return ok();
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_pack");
  }
}

int32_t moe_unpack(int32_t fmt, const uint8_t* src, int64_t src_bytes, int8_t* trits, uint16_t* scales,
                   int64_t n) {
  try {
    if (!known_fmt(fmt)) return bad_fmt(fmt);
    if (n < 0 || n % 128) return fail(MOE_E_SHAPE, "weight count %lld is not a multiple of 128", (long long)n);
    if (n > 0 && (!trits || !scales || !src)) return fail(MOE_E_ARG, "NULL pointer");
    const int64_t need = moe_packed_bytes(fmt, n);
    if (src_bytes < need)
      return fail(MOE_E_SPACE, "container holds %lld bytes, %lld needed", (long long)src_bytes, (long long)need);
    const int64_t nb = n / 128;
    if (fmt == MOE_PQ2_0) {
      for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = src + b * 34;
        for (int j = 0; j < 32; ++j) {
          for (int i = 0; i < 4; ++i) {
            const uint32_t c = (blk[j] >> (2 * i)) & 3u;
            if (c == 2)
              return fail(MOE_E_CODE, "invalid 2-bit code 10 in group %lld, byte %d", (long long)b, j);
            trits[b * 128 + 4 * j + i] = c == 3 ? -1 : (int8_t)c;
          }
        }
        scales[b] = (uint16_t)(blk[32] | (blk[33] << 8));
        if (!finite_f16(scales[b])) return fail(MOE_E_NONFINITE, "non-finite fp16 scale in group %lld", (long long)b);
      }
    } else {
      for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = src + b * 28;
        for (int j = 0; j < 26; ++j) {
          const int nd = j < 24 ? 5 : 4;
          const uint32_t lim = j < 24 ? 243u : 81u;
          if (blk[j] >= lim)
            return fail(MOE_E_CODE, "base-3 %s byte %d > %u in group %lld, byte %d", j < 24 ? "data" : "tail",
                        (int)blk[j], lim - 1, (long long)b, j);
          uint32_t v = blk[j];
          const int base = j < 24 ? 5 * j : 120 + 4 * (j - 24);
          for (int i = 0; i < nd; ++i) {
            const uint32_t dgt = v % 3;
            v /= 3;
            trits[b * 128 + base + i] = dgt == 2 ? -1 : (int8_t)dgt;
          }
        }
        scales[b] = (uint16_t)(blk[26] | (blk[27] << 8));
        if (!finite_f16(scales[b])) return fail(MOE_E_NONFINITE, "non-finite fp16 scale in group %lld", (long long)b);
      }
    }
    return ok();
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in moe_unpack");
  }
}

// Block (row n, group g) of a [rows x cols] container: row-major index n G + g,
// tile-major index ((n / 16) G + g) 16 + n % 16, with G = cols / 128.
static int32_t retile(int32_t fmt, const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                      int64_t dst_bytes, bool to_tiles) {
  try {
    if (!known_fmt(fmt)) return bad_fmt(fmt);
    if (rows < 0 || rows % 16 || cols < 0 || cols % 128)
      return fail(MOE_E_SHAPE, "a %lld x %lld container needs rows %% 16 == 0 and cols %% 128 == 0",
                  (long long)rows, (long long)cols);
    if (rows > 0 && cols > 0 && (!src || !dst)) return fail(MOE_E_ARG, "NULL pointer");
    const int64_t bb = moe_block_bytes(fmt), G = cols / 128, bytes = rows * G * bb;
    if (dst_bytes < bytes)
      return fail(MOE_E_SPACE, "destination holds %lld bytes, %lld needed", (long long)dst_bytes, (long long)bytes);
    if (bytes > 0 && src < dst + bytes && dst < src + bytes) return fail(MOE_E_ARG, "src and dst overlap");
    for (int64_t n = 0; n < rows; ++n)
      for (int64_t g = 0; g < G; ++g) {
        const int64_t plain = n * G + g, tiled = ((n / 16) * G + g) * 16 + n % 16;
        std::memcpy(dst + (to_tiles ? tiled : plain) * bb, src + (to_tiles ? plain : tiled) * bb, (size_t)bb);
      }
    return ok();
  } catch (...) {
    return fail(MOE_E_ARG, "internal error in the container reorder");
  }
}

int32_t moe_tile_container(int32_t fmt, const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                           int64_t dst_bytes) {
  return retile(fmt, src, rows, cols, dst, dst_bytes, true);
}

int32_t moe_untile_container(int32_t fmt, const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                             int64_t dst_bytes) {
  return retile(fmt, src, rows, cols, dst, dst_bytes, false);
}

}  // extern "C"
