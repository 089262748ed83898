// Quantized load cache: file header and SHA-256 (host code).  Internal.
#pragma once
#include <cstddef>
#include <cstdint>
#include <string>

namespace qd {

class Sha256 {
 public:
  Sha256();
  void update(const void* data, size_t n);
  void final(uint8_t out[32]);

 private:
  uint32_t h_[8];
  uint8_t buf_[64];
  size_t fill_ = 0;
  uint64_t total_ = 0;
};

// 128-byte little-endian header, then the payload: the device arena's quantized regions
// in a fixed order (embedding codes, embedding scales, final gain, then per layer q|k|v
// codes and scales, O, gate/up (16-row interleave), down, the four gains)
// digest of a payload: SHA-256 over the concatenated SHA-256 digests of its consecutive
// CACHE_HASH_CHUNK-byte chunks (the last one shorter), the chunks hashed on several threads
constexpr uint64_t CACHE_HASH_CHUNK = uint64_t(16) << 20;
void chunked_sha256(const void* data, uint64_t n, uint8_t out[32]);

struct CacheHeader {
  char magic[8];            // "QDI8WCV1"
  uint32_t version;         // 2 (the chunked payload digest)
  uint32_t header_bytes;    // 128
  uint64_t payload_bytes;
  uint32_t dims[9];         // hidden, layers, heads, kv heads, head_dim, intermediate, vocab,
                            // rms_eps bits, rope_theta bits
  uint8_t source_digest[32];
  uint8_t payload_sha256[32];  // chunked_sha256 of the payload
  uint8_t pad[4];
};
static_assert(sizeof(CacheHeader) == 128, "cache header is 128 bytes");

// every field of h that differs from want (magic first), "" when the gate passes on the
// header; the payload hash is checked separately
std::string cache_header_problems(const CacheHeader& h, const CacheHeader& want);

}  // namespace qd
