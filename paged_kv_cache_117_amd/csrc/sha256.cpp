// SHA-256 as FIPS 180-4 defines it.  The round constants are the first 32
// bits of the fractional parts of the cube roots of the first 64 primes and
// the initial hash value those of the square roots of the first 8 primes;
// both are computed here, exactly, with integer roots (floor of the root of
// p * 2^96, resp. p * 2^64, keeps 32 fractional bits) rather than written out.
#include "sha256.h"

#include <cstring>

namespace pa {
namespace {

using u128 = unsigned __int128;

// floor(x^(1/k)) for k = 2 or 3, by bisection (x < 2^110).
uint64_t iroot(u128 x, int k) {
  uint64_t lo = 0, hi = (uint64_t)1 << 37;
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    u128 p = (u128)mid * mid;
    if (k == 3) p *= mid;
    if (p <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

struct Constants {
  uint32_t k[64];
  uint32_t h0[8];
  Constants() {
    int n = 0;
    for (uint32_t p = 2; n < 64; ++p) {
      bool prime = true;
      for (uint32_t d = 2; d * d <= p; ++d)
        if (p % d == 0) prime = false;
      if (!prime) continue;
      k[n] = (uint32_t)iroot((u128)p << 96, 3);  // low 32 bits = fractional part
      if (n < 8) h0[n] = (uint32_t)iroot((u128)p << 64, 2);
      ++n;
    }
  }
};

const Constants& consts() {
  static const Constants c;
  return c;
}

inline uint32_t rotr(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }

}  // namespace

Sha256::Sha256() { std::memcpy(h_, consts().h0, sizeof(h_)); }

void Sha256::block(const uint8_t* p) {
  const uint32_t* K = consts().k;
  uint32_t w[64];
  for (int i = 0; i < 16; ++i)
    w[i] = (uint32_t)p[4 * i] << 24 | (uint32_t)p[4 * i + 1] << 16 | (uint32_t)p[4 * i + 2] << 8 | p[4 * i + 3];
  for (int i = 16; i < 64; ++i) {
    const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
    const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
    w[i] = w[i - 16] + s0 + w[i - 7] + s1;
  }
  uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6], h = h_[7];
  for (int i = 0; i < 64; ++i) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = h + S1 + ch + K[i] + w[i];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
    h = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  h_[0] += a;
  h_[1] += b;
  h_[2] += c;
  h_[3] += d;
  h_[4] += e;
  h_[5] += f;
  h_[6] += g;
  h_[7] += h;
}

void Sha256::update(const void* data, size_t n) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  bits_ += (uint64_t)n * 8;
  while (n > 0) {
    const size_t take = n < 64 - fill_ ? n : 64 - fill_;
    std::memcpy(buf_ + fill_, p, take);
    fill_ += take;
    p += take;
    n -= take;
    if (fill_ == 64) {
      block(buf_);
      fill_ = 0;
    }
  }
}

Digest Sha256::finish() {
  // Padding: 0x80, zeros up to 56 bytes modulo 64, the bit length (big-endian).
  const uint64_t bits = bits_;
  uint8_t pad[72] = {0x80};
  const size_t nz = (fill_ < 56 ? 56 - fill_ : 120 - fill_);  // 0x80 plus zeros
  for (int i = 0; i < 8; ++i) pad[nz + i] = (uint8_t)(bits >> (56 - 8 * i));
  update(pad, nz + 8);
  Digest d;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) d[4 * i + j] = (uint8_t)(h_[i] >> (24 - 8 * j));
  return d;
}

}  // namespace pa
