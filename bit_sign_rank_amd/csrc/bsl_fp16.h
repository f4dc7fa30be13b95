// Host-side IEEE binary16 conversions of libbitstack_linear (folding an input-channel
// scale into V at load).  Plain C++, no HIP: also compiled alone by the CPU tests.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstring>

namespace bsl {

// IEEE binary16 <-> double on the host (for folding an input-channel scale into V).
inline double fp16_to_double(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double v;
  if (e == 0) v = std::ldexp((double)f, -24);       // zero / subnormal
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + f), e - 25);  // 1.f * 2^(e - 15)
  return (h & 0x8000) ? -v : v;
}

// Round a double to the nearest binary16, ties to even, from its bits.  False if the
// result would be infinite (or v is not finite).
inline bool double_to_fp16(double v, uint16_t* out) {
  uint64_t b;
  std::memcpy(&b, &v, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000);
  const int be = (int)((b >> 52) & 0x7FF);
  if (be == 0x7FF) return false;
  if (be == 0) {  // zero or a double subnormal: far below half the least fp16 subnormal
    *out = sign;
    return true;
  }
  const int e = be - 1023;                                       // v = 1.m * 2^e
  const uint64_t sig = (b & ((1ull << 52) - 1)) | (1ull << 52);  // 53 significant bits
  // keep 11 bits for a normal result (e >= -14), fewer for a subnormal (units of 2^-24)
  const int shift = e >= -14 ? 42 : 42 + (-14 - e);
  if (shift > 53) {  // |v| < 2^-25: rounds to zero
    *out = sign;
    return true;
  }
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1), halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1))) ++q;
  uint32_t h;
  if (e >= -14) {
    int ee = e;
    if (q == 2048) {  // rounded up to the next power of two
      q = 1024;
      ++ee;
    }
    if (ee > 15) return false;
    h = ((uint32_t)(ee + 15) << 10) | (uint32_t)(q - 1024);
  } else {
    h = (uint32_t)q;  // 0..1024; 1024 is the encoding of 2^-14, the least normal
  }
  *out = sign | (uint16_t)h;
  return true;
}

}  // namespace bsl
