// Quantized load cache ("Model-agnostic LLM inference", section "The quantized load
// cache"): the exact post-quantization device bytes (int8 codes, per-row fp32 scales and
// fp32 gains) persisted to a file, restored instead of re-quantizing, behind a validity
// gate of magic + dims + a digest of the source checkpoint + exact length.  This build
// adds a digest of the payload to the gate, so a damaged file is refused too: the SHA-256
// of the SHA-256 digests of its consecutive 16 MiB chunks, which several threads compute
// at once (a single SHA-256 over 0.6 GB takes longer than the rest of the restore).
//
// SHA-256 follows FIPS 180-4; its round constants and initial hash are derived here from
// their definition (the first 32 fractional bits of the cube roots of the first 64 primes
// and of the square roots of the first 8) and corrected to the exact integer value.
#include "qd_cache.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

namespace qd {
namespace {

// floor(frac(p^(1/n)) * 2^32), exact: a long double estimate corrected by integer tests
uint32_t frac_root_bits(uint32_t p, int n) {
  long double r = n == 2 ? sqrtl((long double)p) : cbrtl((long double)p);
  const uint64_t ip = (uint64_t)r;
  // x = floor(p^(1/n) * 2^32) satisfies x^n <= p * 2^(32n) < (x + 1)^n
  unsigned __int128 x = (unsigned __int128)(r * 4294967296.0L);
  auto pw = [&](unsigned __int128 v) {
    unsigned __int128 t = v;
    for (int i = 1; i < n; ++i) t *= v;
    return t;
  };
  const unsigned __int128 target = (unsigned __int128)p << (32 * n);
  while (pw(x) > target) --x;
  while (pw(x + 1) <= target) ++x;
  (void)ip;
  return (uint32_t)(x & 0xFFFFFFFFu);
}

struct ShaConst {
  uint32_t k[64], h0[8];
  ShaConst() {
    int found = 0;
    for (uint32_t c = 2; found < 64; ++c) {
      bool prime = true;
      for (uint32_t q = 2; q * q <= c; ++q)
        if (c % q == 0) { prime = false; break; }
      if (!prime) continue;
      k[found] = frac_root_bits(c, 3);
      if (found < 8) h0[found] = frac_root_bits(c, 2);
      ++found;
    }
  }
};
const ShaConst& sha_const() {
  static const ShaConst c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void sha_block(uint32_t h[8], const uint8_t* blk, const uint32_t* K) {
  uint32_t w[64];
  for (int i = 0; i < 16; ++i)
    w[i] = (uint32_t)blk[4 * i] << 24 | (uint32_t)blk[4 * i + 1] << 16 | (uint32_t)blk[4 * i + 2] << 8 | blk[4 * i + 3];
  for (int i = 16; i < 64; ++i) {
    const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
    const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
    w[i] = w[i - 16] + s0 + w[i - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int i = 0; i < 64; ++i) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + K[i] + w[i];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + mj;
    hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

}  // namespace

Sha256::Sha256() {
  std::memcpy(h_, sha_const().h0, sizeof(h_));
}

void Sha256::update(const void* data, size_t n) {
  const uint8_t* p = (const uint8_t*)data;
  const uint32_t* K = sha_const().k;
  total_ += n;
  if (fill_) {
    const size_t take = std::min(n, (size_t)64 - fill_);
    std::memcpy(buf_ + fill_, p, take);
    fill_ += take; p += take; n -= take;
    if (fill_ == 64) { sha_block(h_, buf_, K); fill_ = 0; }
  }
  for (; n >= 64; p += 64, n -= 64) sha_block(h_, p, K);
  if (n) { std::memcpy(buf_, p, n); fill_ = n; }
}

void Sha256::final(uint8_t out[32]) {
  const uint64_t bits = (uint64_t)total_ * 8;
  const uint8_t one = 0x80, zero = 0;
  update(&one, 1);
  while (fill_ != 56) update(&zero, 1);
  uint8_t len[8];
  for (int i = 0; i < 8; ++i) len[i] = (uint8_t)(bits >> (56 - 8 * i));
  update(len, 8);
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h_[i] >> (24 - 8 * j));
}

void chunked_sha256(const void* data, uint64_t n, uint8_t out[32]) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  const uint64_t chunks = n == 0 ? 0 : (n + CACHE_HASH_CHUNK - 1) / CACHE_HASH_CHUNK;
  std::vector<uint8_t> sums(chunks * 32);
  auto hash_chunk = [&](uint64_t c) {
    const uint64_t at = c * CACHE_HASH_CHUNK;
    Sha256 s;
    s.update(p + at, std::min<uint64_t>(CACHE_HASH_CHUNK, n - at));
    s.final(&sums[c * 32]);
  };
  // every chunk is hashed independently, on up to 16 threads
  const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  const uint64_t nthreads = std::min<uint64_t>(std::min<uint64_t>(hw, 16), chunks);
  std::atomic<uint64_t> next{0};
  auto worker = [&]() {
    for (uint64_t c = next++; c < chunks; c = next++) hash_chunk(c);
  };
  std::vector<std::thread> pool;
  for (uint64_t t = 1; t < nthreads; ++t) pool.emplace_back(worker);
  worker();
  for (auto& t : pool) t.join();
  Sha256 top;
  top.update(sums.data(), sums.size());
  top.final(out);
}

std::string cache_header_problems(const CacheHeader& h, const CacheHeader& want) {
  std::string p;
  auto add = [&](const std::string& s) { p += (p.empty() ? "" : "; ") + s; };
  if (std::memcmp(h.magic, want.magic, sizeof(h.magic)) != 0) return "not a quantized weight cache (magic)";
  if (h.version != want.version) add("format version " + std::to_string(h.version));
  if (h.header_bytes != want.header_bytes) add("header size " + std::to_string(h.header_bytes));
  const char* names[9] = {"hidden", "n_layers", "n_heads", "n_kv_heads", "head_dim", "intermediate",
                          "vocab", "rms_eps", "rope_theta"};
  for (int i = 0; i < 9; ++i)
    if (h.dims[i] != want.dims[i]) add(std::string(names[i]) + " differs");
  if (std::memcmp(h.source_digest, want.source_digest, 32) != 0) add("source checkpoint digest differs");
  if (h.payload_bytes != want.payload_bytes) add("payload length " + std::to_string(h.payload_bytes));
  return p;
}

}  // namespace qd
