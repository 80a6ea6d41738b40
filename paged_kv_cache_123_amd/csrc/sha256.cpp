// SHA-256 as FIPS 180-4 defines it (sections 4.1.2, 4.2.2, 5.1.1, 5.3.3,
// 6.2.2).  The constants are derived from their definition rather than
// typed in: K[t] is the first 32 bits of the fractional part of the cube root
// of the t-th prime (t < 64), H0 those of the square roots of the first eight
// primes, both computed exactly with integer roots.
#include "sha256.h"

#include <cstring>

namespace pa {
namespace {

using u128 = unsigned __int128;

// floor(n^(1/k)) for k = 2 or 3 by bisection on 128-bit integers
uint64_t iroot(u128 n, int k) {
  uint64_t lo = 0, hi = uint64_t(1) << 40;
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    u128 p = mid;
    for (int i = 1; i < k; ++i) p *= mid;
    if (p <= n) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct Constants {
  uint32_t k[64];
  uint32_t h0[8];
  Constants() {
    int found = 0;
    for (uint32_t c = 2; found < 64; ++c) {
      bool prime = true;
      for (uint32_t d = 2; d * d <= c; ++d)
        if (c % d == 0) { prime = false; break; }
      if (!prime) continue;
      // frac(p^(1/3)) * 2^32 = floor((p * 2^96)^(1/3)) mod 2^32
      k[found] = static_cast<uint32_t>(iroot(static_cast<u128>(c) << 96, 3));
      if (found < 8) h0[found] = static_cast<uint32_t>(iroot(static_cast<u128>(c) << 64, 2));
      ++found;
    }
  }
};

const Constants& constants() {
  static const Constants c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void compress(uint32_t h[8], const uint8_t block[64], const Constants& c) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t(block[4 * t]) << 24) | (uint32_t(block[4 * t + 1]) << 16) |
           (uint32_t(block[4 * t + 2]) << 8) | uint32_t(block[4 * t + 3]);
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = w[t - 16] + s0 + w[t - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], cc = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t big1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + big1 + ch + c.k[t] + w[t];
    const uint32_t big0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & cc) ^ (b & cc);
    const uint32_t t2 = big0 + maj;
    hh = g; g = f; f = e; e = d + t1; d = cc; cc = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += cc; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

}  // namespace

Digest sha256(const uint8_t* const* parts, const size_t* sizes, int num_parts) {
  const Constants& c = constants();
  uint32_t h[8];
  std::memcpy(h, c.h0, sizeof h);
  uint8_t buf[64];
  size_t fill = 0;
  uint64_t total = 0;
  for (int i = 0; i < num_parts; ++i) {
    const uint8_t* p = parts[i];
    size_t n = sizes[i];
    total += n;
    while (n > 0) {
      const size_t take = n < 64 - fill ? n : 64 - fill;
      std::memcpy(buf + fill, p, take);
      fill += take;
      p += take;
      n -= take;
      if (fill == 64) {
        compress(h, buf, c);
        fill = 0;
      }
    }
  }
  // padding: a 1 bit, zeros, the message length in bits (big-endian 64-bit)
  buf[fill++] = 0x80;
  if (fill > 56) {
    std::memset(buf + fill, 0, 64 - fill);
    compress(h, buf, c);
    fill = 0;
  }
  std::memset(buf + fill, 0, 56 - fill);
  const uint64_t bits = total * 8;
  for (int i = 0; i < 8; ++i) buf[56 + i] = static_cast<uint8_t>(bits >> (56 - 8 * i));
  compress(h, buf, c);
  Digest out;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = static_cast<uint8_t>(h[i] >> (24 - 8 * j));
  return out;
}

}  // namespace pa
