// SHA-256 from FIPS 180-4: constants of section 4.2.2 and 5.3.3, padding of
// section 5.1.1, computation of section 6.2.2.
#include "pa_sha256.h"

#include <cstring>

namespace pa {
namespace {

// first 32 bits of the fractional parts of the cube roots of the first 64
// primes (section 4.2.2)
constexpr uint32_t kRound[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4,
    0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe,
    0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f,
    0x4a7484aa, 0x5cb0a9dc, 0x76f988da, 0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7,
    0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc,
    0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
    0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070, 0x19a4c116,
    0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7,
    0xc67178f2};

// first 32 bits of the fractional parts of the square roots of the first 8
// primes (section 5.3.3)
constexpr uint32_t kInit[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                               0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }
inline uint32_t big_sigma0(uint32_t x) { return rotr(x, 2) ^ rotr(x, 13) ^ rotr(x, 22); }
inline uint32_t big_sigma1(uint32_t x) { return rotr(x, 6) ^ rotr(x, 11) ^ rotr(x, 25); }
inline uint32_t small_sigma0(uint32_t x) { return rotr(x, 7) ^ rotr(x, 18) ^ (x >> 3); }
inline uint32_t small_sigma1(uint32_t x) { return rotr(x, 17) ^ rotr(x, 19) ^ (x >> 10); }
inline uint32_t choose(uint32_t x, uint32_t y, uint32_t z) { return (x & y) ^ (~x & z); }
inline uint32_t majority(uint32_t x, uint32_t y, uint32_t z) {
  return (x & y) ^ (x & z) ^ (y & z);
}

}  // namespace

Sha256::Sha256() { std::memcpy(h_, kInit, sizeof(h_)); }

void Sha256::compress(const uint8_t block[64]) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t(block[4 * t]) << 24) | (uint32_t(block[4 * t + 1]) << 16) |
           (uint32_t(block[4 * t + 2]) << 8) | uint32_t(block[4 * t + 3]);
  for (int t = 16; t < 64; ++t)
    w[t] = small_sigma1(w[t - 2]) + w[t - 7] + small_sigma0(w[t - 15]) + w[t - 16];
  uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3];
  uint32_t e = h_[4], f = h_[5], g = h_[6], h = h_[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t t1 = h + big_sigma1(e) + choose(e, f, g) + kRound[t] + w[t];
    const uint32_t t2 = big_sigma0(a) + majority(a, b, c);
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

void Sha256::update(const void* data, size_t len) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  total_ += len;
  if (buf_len_ > 0) {
    const size_t take = len < 64 - buf_len_ ? len : 64 - buf_len_;
    std::memcpy(buf_ + buf_len_, p, take);
    buf_len_ += take;
    p += take;
    len -= take;
    if (buf_len_ < 64) return;
    compress(buf_);
    buf_len_ = 0;
  }
  for (; len >= 64; p += 64, len -= 64) compress(p);
  std::memcpy(buf_, p, len);
  buf_len_ = len;
}

void Sha256::finish(uint8_t digest[32]) {
  // padding: a one bit, zeros up to 56 bytes mod 64, the bit length (64-bit
  // big-endian)
  const uint64_t bits = total_ * 8;
  buf_[buf_len_++] = 0x80;
  if (buf_len_ > 56) {
    std::memset(buf_ + buf_len_, 0, 64 - buf_len_);
    compress(buf_);
    buf_len_ = 0;
  }
  std::memset(buf_ + buf_len_, 0, 56 - buf_len_);
  for (int i = 0; i < 8; ++i) buf_[56 + i] = uint8_t(bits >> (56 - 8 * i));
  compress(buf_);
  for (int i = 0; i < 8; ++i) {
    digest[4 * i] = uint8_t(h_[i] >> 24);
    digest[4 * i + 1] = uint8_t(h_[i] >> 16);
    digest[4 * i + 2] = uint8_t(h_[i] >> 8);
    digest[4 * i + 3] = uint8_t(h_[i]);
  }
}

void sha256(const void* data, size_t len, uint8_t digest[32]) {
  Sha256 s;
  s.update(data, len);
  s.finish(digest);
}

}  // namespace pa
