// SHA-256 (FIPS 180-4), host only: the chained block hash of the prefix cache.
#pragma once

#include <array>
#include <cstddef>
#include <cstdint>

namespace pa {

using Digest = std::array<uint8_t, 32>;

class Sha256 {
 public:
  Sha256();
  void update(const void* data, size_t n);
  Digest finish();  // the object is spent afterwards

 private:
  void block(const uint8_t* p);
  uint32_t h_[8];
  uint8_t buf_[64];
  size_t fill_ = 0;
  uint64_t bits_ = 0;
};

}  // namespace pa
