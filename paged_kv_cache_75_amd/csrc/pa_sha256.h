// SHA-256 as defined in FIPS 180-4 (Secure Hash Standard), section 6.2:
// 512-bit message blocks, the eight-word state, the 64-entry message
// schedule and the compression rounds.  Host code only.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pa {

class Sha256 {
 public:
  Sha256();
  void update(const void* data, size_t len);
  void finish(uint8_t digest[32]);   // the object is spent afterwards

 private:
  void compress(const uint8_t block[64]);
  uint32_t h_[8];
  uint8_t buf_[64];
  size_t buf_len_ = 0;
  uint64_t total_ = 0;               // message length in bytes
};

void sha256(const void* data, size_t len, uint8_t digest[32]);

}  // namespace pa
