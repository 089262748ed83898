// Host-code harness for the AddressSanitizer + UndefinedBehaviorSanitizer build of the
// library's host side (qd_api.hip compiled for the host only, qd_cache.cpp).  It drives the
// C ABI through every path that returns before GPU work: the architecture gates
// ("Model-agnostic LLM inference", sections "Supported models" and "Errors"), buffer
// sizing and limits, SHA-256 (FIPS 180-4) and the quantized load cache's file gate
// ("The quantized load cache") on well-formed, truncated and damaged files, and every entry
// point's argument checks.  Exit status 0 and a final "ok" line mean every expectation held
// and the sanitizers reported nothing (they abort the process on the first report).
#include "qd.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

static int failures = 0;
#define EXPECT(cond, what)                                         \
  do {                                                             \
    if (!(cond)) {                                                 \
      std::fprintf(stderr, "FAILED: %s (%s)\n", what, qd_last_error()); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static std::string hex(const uint8_t* d, int n) {
  static const char* h = "0123456789abcdef";
  std::string s;
  for (int i = 0; i < n; ++i) { s += h[d[i] >> 4]; s += h[d[i] & 15]; }
  return s;
}

static qd_model_shape tiny() {
  qd_model_shape s{};
  s.hidden = 128; s.n_layers = 2; s.n_heads = 4; s.n_kv_heads = 2; s.head_dim = 32;
  s.intermediate = 384; s.vocab = 1024; s.rms_eps = 1e-6f; s.rope_theta = 1e6f;
  s.tie_word_embeddings = 1; s.attention_bias = 0;
  return s;
}

// payload bytes of the quantized cache for a shape, from the layout in qd.h
static uint64_t payload_bytes(const qd_model_shape& s) {
  const uint64_t d = s.hidden, L = s.n_layers, H = s.n_heads, KV = s.n_kv_heads, D = s.head_dim,
                 I = s.intermediate, V = s.vocab, nqkv = H * D + 2 * KV * D;
  const uint64_t per_layer = nqkv * d + 4 * nqkv + d * H * D + 4 * d + 2 * I * d + 8 * I + d * I +
                             4 * d + 4 * d + 4 * d + 4 * D + 4 * D;
  return V * d + 4 * V + 4 * d + L * per_layer;
}

// the documented payload digest: SHA-256 over the SHA-256 digests of 16 MiB chunks
static void payload_digest(const std::vector<uint8_t>& p, uint8_t out[32]) {
  const uint64_t chunk = uint64_t(16) << 20;
  std::vector<uint8_t> sums;
  for (uint64_t at = 0; at < p.size(); at += chunk) {
    uint8_t d[32];
    const uint64_t n = p.size() - at < chunk ? p.size() - at : chunk;
    qd_sha256(p.data() + at, n, d);
    sums.insert(sums.end(), d, d + 32);
  }
  qd_sha256(sums.data(), sums.size(), out);
}

static void write_cache(const char* path, const qd_model_shape& s, const uint8_t digest[32],
                        const std::vector<uint8_t>& payload, uint32_t version, long truncate_to) {
  uint8_t hdr[128];
  std::memset(hdr, 0, sizeof(hdr));
  std::memcpy(hdr, "QDI8WCV1", 8);
  const uint32_t hb = 128;
  const uint64_t pb = payload.size();
  std::memcpy(hdr + 8, &version, 4);
  std::memcpy(hdr + 12, &hb, 4);
  std::memcpy(hdr + 16, &pb, 8);
  uint32_t dims[9] = {(uint32_t)s.hidden, (uint32_t)s.n_layers, (uint32_t)s.n_heads,
                      (uint32_t)s.n_kv_heads, (uint32_t)s.head_dim, (uint32_t)s.intermediate,
                      (uint32_t)s.vocab, 0, 0};
  std::memcpy(&dims[7], &s.rms_eps, 4);
  std::memcpy(&dims[8], &s.rope_theta, 4);
  std::memcpy(hdr + 24, dims, 36);
  std::memcpy(hdr + 60, digest, 32);
  payload_digest(payload, hdr + 92);
  std::vector<uint8_t> file(hdr, hdr + 128);
  file.insert(file.end(), payload.begin(), payload.end());
  if (truncate_to >= 0 && (size_t)truncate_to < file.size()) file.resize(truncate_to);
  FILE* f = std::fopen(path, "wb");
  if (!f) { std::perror(path); std::exit(3); }
  std::fwrite(file.data(), 1, file.size(), f);
  std::fclose(f);
}

int main(int argc, char** argv) {
  const std::string dir = argc > 1 ? argv[1] : ".";
  // ---- gates ----
  qd_model_shape s = tiny();
  EXPECT(qd_check_shape(&s) == QD_OK, "tiny shape passes");
  EXPECT(qd_check_shape(nullptr) == QD_ERR_UNSUPPORTED_ARCH, "NULL shape");
  const int bad[][2] = {{0, 100}, {3, 3}, {5, 300}, {4, 20}, {1, 0}, {6, 1}};
  for (auto& b : bad) {
    qd_model_shape t = tiny();
    int32_t* f[] = {&t.hidden, &t.n_layers, &t.n_heads, &t.n_kv_heads, &t.head_dim, &t.intermediate,
                    &t.vocab};
    *f[b[0]] = b[1];
    EXPECT(qd_check_shape(&t) == QD_ERR_UNSUPPORTED_ARCH, "a failing gate");
    EXPECT(std::strlen(qd_last_error()) > 0, "a failing gate is named");
  }
  qd_model_shape nb = tiny();
  nb.tie_word_embeddings = 0; nb.attention_bias = 1; nb.rms_eps = -1.0f;
  EXPECT(qd_check_shape(&nb) == QD_ERR_UNSUPPORTED_ARCH, "several failing gates");
  // ---- sizes and limits ----
  qd_sizes z{};
  const qd_limits lims[] = {{1, 512, 64}, {64, 65536, 4000}, {0, 512, 64}, {65, 512, 64},
                            {1, 65537, 64}, {1, 0, 64}, {1, 512, 0}, {1, 512, 4000001},
                            {1, 512, 2796203}};
  const qd_status want[] = {QD_OK, QD_OK, QD_ERR_INVALID_ARGUMENTS, QD_ERR_INVALID_ARGUMENTS,
                            QD_ERR_CONTEXT_CEILING, QD_ERR_INVALID_ARGUMENTS,
                            QD_ERR_INVALID_ARGUMENTS, QD_ERR_INVALID_ARGUMENTS,
                            QD_ERR_INVALID_ARGUMENTS};
  for (size_t i = 0; i < sizeof(lims) / sizeof(lims[0]); ++i)
    EXPECT(qd_query_sizes(&s, &lims[i], &z) == want[i], "query_sizes limits");
  EXPECT(qd_query_sizes(&s, &lims[0], nullptr) == QD_ERR_INVALID_ARGUMENTS, "query_sizes NULL out");
  EXPECT(qd_query_sizes(&s, nullptr, &z) == QD_ERR_INVALID_ARGUMENTS, "query_sizes NULL limits");
  // ---- SHA-256: the example digests of FIPS 180-4 (appendix examples) ----
  uint8_t d[32];
  qd_sha256("abc", 3, d);
  EXPECT(hex(d, 32) == "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad", "sha256 abc");
  qd_sha256("", 0, d);
  EXPECT(hex(d, 32) == "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855", "sha256 empty");
  const char* m448 = "abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq";
  qd_sha256(m448, std::strlen(m448), d);
  EXPECT(hex(d, 32) == "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1", "sha256 448-bit");
  for (int n = 0; n < 300; ++n) {  // every padding boundary, memory-checked
    std::vector<uint8_t> v(n, (uint8_t)n);
    qd_sha256(v.data(), v.size(), d);
  }
  // ---- the quantized load cache's gate ----
  uint8_t src[32];
  qd_sha256("source checkpoint manifest", 26, src);
  std::vector<uint8_t> payload(payload_bytes(s));
  for (size_t i = 0; i < payload.size(); ++i) payload[i] = (uint8_t)(i * 2654435761u >> 24);
  const std::string good = dir + "/good.cache", bad_path = dir + "/bad.cache";
  write_cache(good.c_str(), s, src, payload, 2, -1);
  EXPECT(qd_check_cache(&s, good.c_str(), src) == QD_OK, "well-formed cache passes");
  const long full = 128 + (long)payload.size();
  const long cuts[] = {0, 1, 100, 127, 128, 129, full / 2, full - 1};
  for (long c : cuts) {
    write_cache(bad_path.c_str(), s, src, payload, 2, c);
    EXPECT(qd_check_cache(&s, bad_path.c_str(), src) == QD_ERR_CACHE_MISS, "truncated cache refused");
  }
  write_cache(bad_path.c_str(), s, src, payload, 1, -1);
  EXPECT(qd_check_cache(&s, bad_path.c_str(), src) == QD_ERR_CACHE_MISS, "old format version refused");
  std::vector<uint8_t> flipped = payload;
  flipped[flipped.size() / 3] ^= 0x10;
  write_cache(bad_path.c_str(), s, src, payload, 2, -1);
  {  // payload damaged after the header was written: the digest no longer matches
    FILE* f = std::fopen(bad_path.c_str(), "r+b");
    std::fseek(f, 128 + (long)(payload.size() / 3), SEEK_SET);
    std::fputc(flipped[flipped.size() / 3], f);
    std::fclose(f);
  }
  EXPECT(qd_check_cache(&s, bad_path.c_str(), src) == QD_ERR_CACHE_MISS, "damaged payload refused");
  {  // one byte appended
    FILE* f = std::fopen(good.c_str(), "ab");
    std::fputc(0, f);
    std::fclose(f);
  }
  EXPECT(qd_check_cache(&s, good.c_str(), src) == QD_ERR_CACHE_MISS, "longer file refused");
  uint8_t other[32];
  qd_sha256("another checkpoint", 18, other);
  write_cache(good.c_str(), s, src, payload, 2, -1);
  EXPECT(qd_check_cache(&s, good.c_str(), other) == QD_ERR_CACHE_MISS, "other source digest refused");
  qd_model_shape s2 = tiny();
  s2.vocab = 1000;
  EXPECT(qd_check_cache(&s2, good.c_str(), src) == QD_ERR_CACHE_MISS, "other dims refused");
  EXPECT(qd_check_cache(&s, (dir + "/missing.cache").c_str(), src) == QD_ERR_CACHE_MISS, "missing file");
  EXPECT(qd_check_cache(&s, nullptr, src) == QD_ERR_INVALID_ARGUMENTS, "NULL path");
  // ---- argument checks of every entry point (no model, no buffers: no GPU work) ----
  qd_model* none = nullptr;
  int32_t ids[4] = {1, 2, 3, 4}, lens[1] = {4}, out_ids[8] = {0}, n_out[1] = {0};
  float us[16];
  EXPECT(qd_prefill(none, 1, ids, ids, lens, nullptr, ids, nullptr) == QD_ERR_INVALID_ARGUMENTS, "prefill");
  EXPECT(qd_prefill_slots(none, 1, ids, ids, ids, lens, nullptr, ids, nullptr) == QD_ERR_INVALID_ARGUMENTS, "prefill_slots");
  EXPECT(qd_decode_step(none, 1, ids, nullptr, ids, nullptr) == QD_ERR_INVALID_ARGUMENTS, "decode_step");
  EXPECT(qd_decode_step_slots(none, 1, ids, ids, nullptr, ids, nullptr) == QD_ERR_INVALID_ARGUMENTS, "decode_step_slots");
  EXPECT(qd_generate_greedy(none, 1, ids, lens, 2, -1, out_ids, n_out, nullptr, nullptr) == QD_ERR_INVALID_ARGUMENTS, "generate");
  qd_sampling sp{0.8f, 40, 0.0f, 0.95f, 1.1f, 0.0f, 0.0f};
  uint64_t seeds[1] = {1};
  EXPECT(qd_sample(none, 1, nullptr, &sp, seeds, us, ids, nullptr) == QD_ERR_INVALID_ARGUMENTS, "sample");
  EXPECT(qd_sample_noalloc(none, 1, nullptr, &sp, seeds, us, ids, nullptr) == QD_ERR_INVALID_ARGUMENTS, "sample_noalloc");
  EXPECT(qd_run_op(none, 0, 0, 1, ids, nullptr, us, nullptr, nullptr) == QD_ERR_INVALID_ARGUMENTS, "run_op");
  EXPECT(qd_profile_kernels(none, 1, 1, us, nullptr) == QD_ERR_INVALID_ARGUMENTS, "profile_kernels");
  EXPECT(qd_set_tuning(none, 0, 1) == QD_ERR_INVALID_ARGUMENTS, "set_tuning");
  int8_t codes[4];
  EXPECT(qd_export_quantized(none, 0, 0, codes, us, nullptr) == QD_ERR_INVALID_ARGUMENTS, "export_quantized");
  EXPECT(qd_save_cache(none, good.c_str(), src, nullptr) == QD_ERR_INVALID_ARGUMENTS, "save_cache");
  qd_free(nullptr);
  // loads that fail their checks before touching the device
  qd_model* m = nullptr;
  qd_buffers nobufs{};
  EXPECT(qd_load_weights(&s, &lims[0], nullptr, &nobufs, nullptr, &m) == QD_ERR_CHECKPOINT_NOT_FOUND, "load without weights");
  qd_layer_f32 layers[2] = {};
  qd_weights_f32 w{nullptr, nullptr, layers};
  EXPECT(qd_load_weights(&s, &lims[0], &w, &nobufs, nullptr, &m) == QD_ERR_CHECKPOINT_NOT_FOUND, "load with NULL tensors");
  EXPECT(std::strstr(qd_last_error(), "embed") != nullptr, "the missing tensors are named");
  EXPECT(qd_load_weights(&nb, &lims[0], &w, &nobufs, nullptr, &m) == QD_ERR_UNSUPPORTED_ARCH, "load of a gated shape");
  EXPECT(qd_load_weights(&s, &lims[4], &w, &nobufs, nullptr, &m) == QD_ERR_CONTEXT_CEILING, "load past the ceiling");
  EXPECT(qd_load_cache(&s, &lims[0], good.c_str(), src, nullptr, nullptr, &m) != QD_OK, "cache load without buffers");
  EXPECT(m == nullptr, "no handle after failed loads");
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
