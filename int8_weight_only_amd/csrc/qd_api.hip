// Host side of the C ABI declared in include/qd.h: shape gates, buffer planning,
// weight loading, and the prefill / decode / generate drivers.
//
// The call shape follows "Model-agnostic LLM inference": gates checked from the
// shape alone before any GPU work (section "Supported models"), named errors that
// list every problem (section "Errors"), one call from prompt ids to generated ids
// with greedy arg-max (section "Notes"), context ceiling 65,536 (section "Long
// context").  Prefill fills the KV cache and decode sweeps the weights once per
// step for all sequences ("LLM inference overview", section "Workload
// characteristics").
#include "qd.h"
#include "qd_common.h"
#include "qd_cache.h"

#include <map>
#include <string>
#include <tuple>
#include <vector>
#include <cstring>
#include <cmath>
#include <cstdio>

using namespace qd;

namespace {

thread_local std::string g_err;

qd_status fail(qd_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct LayerOff {
  size_t qkv_q, qkv_s, o_q, o_s, gu_q, gu_s, dn_q, dn_s;
  size_t in_g, post_g, qn_g, kn_g;
};

struct Plan {
  // weights arena
  size_t emb_q = 0, emb_s = 0, final_g = 0, rope = 0;
  std::vector<LayerOff> L;
  size_t weight_bytes = 0;
  // workspace
  size_t x = 0, h = 0, qkv = 0, attn = 0, act = 0, part_o = 0, part_ml = 0;
  size_t ids = 0, row_slot = 0, row_pos = 0, last_rows = 0, lens = 0, slot_ident = 0, tiles = 0;
  size_t slot_map = 0;  // [max_batch] KV slot of each row of a slot-addressed call
  size_t tok_counts = 0, draws = 0, seeds = 0, samp_z = 0;  // sampler state and scratch
  size_t smp_rowmax = 0, smp_hist = 0, smp_ncand = 0, smp_cand = 0;
  size_t pos = 0, next_ids = 0, lm_keys = 0, att_cnt = 0, sk_cnt = 0, done = 0, step = 0, out_ids = 0;
  size_t gemm_part = 0;
  size_t ws_bytes = 0;
  size_t kv_bytes = 0;
  size_t kv_layer_elems = 0;  // bf16 elements of K (or V) per layer
  int mmax = 0;
  int nsplit_cap = 0;
  uint64_t packed = 0;
};

struct Dims {
  int d, L, H, KV, D, I, V, G, HD, KVD, NQKV;
};

Dims dims_of(const qd_model_shape& s) {
  Dims d;
  d.d = s.hidden; d.L = s.n_layers; d.H = s.n_heads; d.KV = s.n_kv_heads; d.D = s.head_dim;
  d.I = s.intermediate; d.V = s.vocab; d.G = s.n_kv_heads > 0 ? s.n_heads / s.n_kv_heads : 0;
  d.HD = s.n_heads * s.head_dim; d.KVD = s.n_kv_heads * s.head_dim;
  d.NQKV = d.HD + 2 * d.KVD;
  return d;
}

std::string gate_problems(const qd_model_shape* s) {
  std::string p;
  auto add = [&](const std::string& m) { p += (p.empty() ? "" : "; ") + m; };
  if (!s) return "shape is NULL";
  const char* names[] = {"hidden_size", "num_hidden_layers", "num_attention_heads",
                         "num_key_value_heads", "head_dim", "intermediate_size", "vocab_size"};
  const int vals[] = {s->hidden, s->n_layers, s->n_heads, s->n_kv_heads, s->head_dim,
                      s->intermediate, s->vocab};
  bool sizes_ok = true;
  for (int i = 0; i < 7; ++i)
    if (vals[i] <= 0) {
      add(std::string(names[i]) + "=" + std::to_string(vals[i]) + " must be > 0");
      sizes_ok = false;
    }
  // gates of the pages ("Supported models")
  if (s->n_kv_heads > 0 && s->n_heads % s->n_kv_heads != 0)
    add("num_attention_heads (" + std::to_string(s->n_heads) + ") % num_key_value_heads (" +
        std::to_string(s->n_kv_heads) + ") != 0");
  if (s->hidden % 32 != 0) add("hidden_size " + std::to_string(s->hidden) + " not divisible by 32");
  if (s->intermediate % 32 != 0)
    add("intermediate_size " + std::to_string(s->intermediate) + " not divisible by 32");
  if (((long long)s->n_heads * s->head_dim) % 32 != 0)
    add("num_attention_heads * head_dim = " + std::to_string((long long)s->n_heads * s->head_dim) +
        " not divisible by 32");
  if (!s->tie_word_embeddings) add("tie_word_embeddings must be true");
  if (s->attention_bias) add("attention_bias must be false");
  // gates of this library's kernels
  if (sizes_ok) {
    const int D = s->head_dim;
    if (D < 32 || D > 256 || (D & (D - 1)) != 0)
      add("head_dim " + std::to_string(D) + " must be a power of two in [32, 256] (kernel limit)");
    if (s->vocab < 2) add("vocab_size must be >= 2");
    if (s->n_kv_heads > 0 && s->n_heads % s->n_kv_heads == 0 && s->n_heads / s->n_kv_heads > 8)
      add("num_attention_heads / num_key_value_heads > 8 (kernel limit)");
  }
  if (!(s->rms_eps > 0.0f)) add("rms_norm_eps must be > 0");
  if (!(s->rope_theta > 0.0f)) add("rope_theta must be > 0");
  return p;
}

qd_status check_limits(const qd_limits* lim) {
  if (!lim) return fail(QD_ERR_INVALID_ARGUMENTS, "limits is NULL");
  if (lim->max_ctx > QD_MAX_CONTEXT)
    return fail(QD_ERR_CONTEXT_CEILING, "max_ctx " + std::to_string(lim->max_ctx) +
                                            " exceeds the context ceiling " +
                                            std::to_string(QD_MAX_CONTEXT));
  std::string p;
  if (lim->max_batch < 1 || lim->max_batch > 64) p += "max_batch must be in [1, 64]; ";
  if (lim->max_ctx < 1) p += "max_ctx must be >= 1; ";
  // one prefill attention work-group row per 64 prompt rows: at most 65535 of them
  if (lim->max_prefill_tokens < 1 || lim->max_prefill_tokens > 4000000)
    p += "max_prefill_tokens must be in [1, 4000000]; ";
  if (!p.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, p);
  return QD_OK;
}

// The prefill GEMM addresses each operand through one buffer resource with 32-bit byte
// offsets (and reads zero at offset 2^31): every [M, width] bf16 operand it reads or writes
// must stay below 2 GiB, so max_prefill_tokens is bounded by the widest row the shape has.
std::string prefill_bound_problem(const qd_model_shape& s, const qd_limits& lim) {
  const Dims d = dims_of(s);
  const long long widest = std::max(std::max((long long)d.d, (long long)d.I),
                                     std::max((long long)d.NQKV, (long long)d.HD));
  const long long rows = std::max((long long)lim.max_prefill_tokens, (long long)lim.max_batch);
  const long long cap = ((1ll << 31) - 1) / (2 * widest);
  if (rows > cap)
    return "max_prefill_tokens " + std::to_string(lim.max_prefill_tokens) + " exceeds " +
           std::to_string(cap) + " for this shape (prefill operands are addressed with 32-bit " +
           "offsets: tokens x widest row (" + std::to_string(widest) + ") x 2 bytes < 2 GiB)";
  return "";
}

Plan make_plan(const qd_model_shape& s, const qd_limits& lim) {
  const Dims d = dims_of(s);
  Plan P;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  P.emb_q = take((size_t)d.V * d.d);
  P.emb_s = take((size_t)d.V * 4);
  P.final_g = take((size_t)d.d * 4);
  P.L.resize(d.L);
  for (int l = 0; l < d.L; ++l) {
    LayerOff& o = P.L[l];
    o.qkv_q = take((size_t)d.NQKV * d.d);
    o.qkv_s = take((size_t)d.NQKV * 4);
    o.o_q = take((size_t)d.d * d.HD);
    o.o_s = take((size_t)d.d * 4);
    o.gu_q = take((size_t)2 * d.I * d.d);
    o.gu_s = take((size_t)2 * d.I * 4);
    o.dn_q = take((size_t)d.d * d.I);
    o.dn_s = take((size_t)d.d * 4);
    o.in_g = take((size_t)d.d * 4);
    o.post_g = take((size_t)d.d * 4);
    o.qn_g = take((size_t)d.D * 4);
    o.kn_g = take((size_t)d.D * 4);
  }
  P.rope = take((size_t)lim.max_ctx * (d.D / 2) * 8);
  P.weight_bytes = off;

  const int B = lim.max_batch;
  const int M = std::max(lim.max_batch, lim.max_prefill_tokens);
  P.mmax = M;
  const int chunks = (lim.max_ctx + ATT_CHUNK - 1) / ATT_CHUNK;
  P.nsplit_cap = std::min(chunks, ATT_MAX_SPLITS);
  off = 0;
  P.x = take((size_t)M * d.d * 2);
  P.h = take((size_t)M * d.d * 2);
  P.qkv = take((size_t)M * d.NQKV * 2);
  P.attn = take((size_t)M * d.HD * 2);
  P.act = take((size_t)M * d.I * 2);
  P.part_o = take((size_t)B * d.H * P.nsplit_cap * d.D * 4);
  P.part_ml = take((size_t)B * d.H * P.nsplit_cap * 2 * 4);
  P.ids = take((size_t)M * 4);
  P.row_slot = take((size_t)M * 4);
  P.row_pos = take((size_t)M * 4);
  P.last_rows = take((size_t)B * 4);
  P.tiles = take((size_t)(M / FLASH_ROWS + B + 1) * 16);
  P.lens = take((size_t)B * 4);
  P.slot_ident = take((size_t)B * 4);
  P.slot_map = take((size_t)B * 4);
  P.tok_counts = take((size_t)B * d.V * 4);
  P.draws = take((size_t)B * 4);
  P.seeds = take((size_t)B * 8);
  P.samp_z = take((size_t)B * d.V * 4);
  P.smp_rowmax = take((size_t)B * 4);
  P.smp_hist = take((size_t)B * 256 * 4);
  P.smp_ncand = take((size_t)B * 4);
  P.smp_cand = take((size_t)B * SMP_CAND_G * 8);
  P.pos = take((size_t)B * 4);
  P.next_ids = take((size_t)B * 4);
  P.lm_keys = take((size_t)B * LM_MAX_GRID * 8);
  P.att_cnt = take((size_t)B * d.KV * 4);
  P.sk_cnt = take((size_t)SKINNY_MAX_TILES * 4);
  P.done = take(64);
  P.step = take(64);
  P.out_ids = take((size_t)B * lim.max_ctx * 4);
  P.gemm_part = take(GEMM_PART_FLOATS * 4);
  P.ws_bytes = off;

  P.kv_layer_elems = (size_t)B * d.KV * lim.max_ctx * d.D;
  P.kv_bytes = (size_t)d.L * 2 * P.kv_layer_elems * 2;

  // int8 codes + one fp32 scale per output row + fp32 gains, tied embedding once
  uint64_t per_layer = 0;
  const int64_t rc[7][2] = {{d.HD, d.d}, {d.KVD, d.d}, {d.KVD, d.d}, {d.d, d.HD},
                            {d.I, d.d},  {d.I, d.d},   {d.d, d.I}};
  for (auto& r : rc) per_layer += (uint64_t)(r[0] * r[1] + 4 * r[0]);
  per_layer += 4ull * (2 * d.d + 2 * d.D);
  P.packed = (uint64_t)d.L * per_layer + (uint64_t)d.V * d.d + 4ull * d.V + 4ull * d.d;
  return P;
}

}  // namespace

struct qd_model {
  qd_model_shape shape;
  qd_limits lim;
  Dims d;
  Plan P;
  char* W = nullptr;   // weights arena
  char* KVb = nullptr; // KV cache
  char* WS = nullptr;  // workspace
  int device = 0;
  hipStream_t cap_stream = nullptr;
  std::map<std::tuple<int, int, int, int>, hipGraphExec_t> graphs;  // (B, nsplit, split_len*16 + waves, steps)
  std::vector<int> host_pos;                                   // mirror of device positions
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  // pinned host staging for prompt ids and prefill metadata: asynchronous uploads read
  // from here, so the source outlives the copy; stage_ev guards reuse
  int* hstage = nullptr;
  size_t hstage_ints = 0;
  hipEvent_t stage_ev = nullptr;
  bool stage_pending = false;
  int attn_max_splits = 64;
  int attn_min_chunks = 1;
  int attn_occupancy = 0;  // attention work-groups per CU the split targets (0: by waves)
  int attn_resident4 = 3;  // four-wave attention work-groups that fit on one CU (measured)
  int attn_waves = 0;  // 0: eight waves only when B x KV heads fill the GPU without splits
  int attn_merge_last = 1;
  void* noalloc_scratch = nullptr;  // this device's address of the sampler's fixed scratch
  int gemm_splits = 0;  // prefill GEMM split-K cap (0: launcher default)
  int gemm_ks = 1;      // prefill GEMMs of few rows may take the k-sliced kernel
  int gemm_rope = 1;    // the q|k|v GEMM may run QK-norm / RoPE in its epilogue (above the k-sliced kernel's rows)
  int flash_rows = 0;   // prefill attention query tile rows: 64, 128, or 0 (by prompt size)
  int skinny_norm = 1;   // batched projections fold the RMSNorm where the shape allows
  int skinny_split = 2;  // 1: never; 2: fewer than 128 channel tiles, over 16 rows; 3: all
  int skinny_xstage = 1; // batched projections load activations row-contiguously via LDS

  template <class T> T* w(size_t off) { return reinterpret_cast<T*>(W + off); }
  template <class T> T* ws(size_t off) { return reinterpret_cast<T*>(WS + off); }
  bf16_t* kcache(int l) { return reinterpret_cast<bf16_t*>(KVb) + (size_t)(2 * l) * P.kv_layer_elems; }
  bf16_t* vcache(int l) { return reinterpret_cast<bf16_t*>(KVb) + (size_t)(2 * l + 1) * P.kv_layer_elems; }
};

#define HIPCHK(expr)                                                                  \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(QD_ERR_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

namespace {

// attention split over positions 0..ctx-1, from the context, the tuning knobs and the
// number of (row, KV head) pairs: work-groups in flight are capped near `occupancy` per CU
// (256 CUs), since more splits only add merge traffic
void attn_split(int ctx, int cap, int max_splits, int min_chunks, int occupancy, int rows_x_kv,
                int* nsplit, int* split_len);

// decode-attention waves per work-group: eight from 64 (row, KV head) pairs up or when the
// context is long (more than ATT_LONG_CTX positions), else four
int attn_waves_for(const qd_model* m, int B, int ctx);
// work-groups per CU the split targets: as many as stay resident (the 8-wave kernel holds
// one per CU, the 4-wave kernel three; measured best at B = 1..32)
int attn_occupancy_for(const qd_model* m, int B, int ctx);

void attn_split(int ctx, int cap, int max_splits, int min_chunks, int occupancy, int rows_x_kv,
                int* nsplit, int* split_len) {
  const int chunks = std::max(1, (ctx + ATT_CHUNK - 1) / ATT_CHUNK);
  max_splits = std::min(max_splits, std::max(1, 256 * occupancy / std::max(1, rows_x_kv)));
  int want = std::max(1, std::min(std::min(chunks, cap), max_splits));
  want = std::max(1, std::min(want, chunks / std::max(1, min_chunks)));
  const int per = (chunks + want - 1) / want;
  *split_len = per * ATT_CHUNK;
  *nsplit = (chunks + per - 1) / per;
}

// LM head + fused arg-max.  One row: the register GEMV normalizes in its prologue.
// Several rows: the rows are RMS-normalized into the h buffer (rows_total rows of x,
// gathered through x_rows when given) and one MFMA sweep of the embedding serves all.
qd_status enqueue_lm_head(qd_model* m, const bf16_t* x, const int* x_rows, int rows_total, int B,
                          float* logits, int* next_ids, bool bump_pos, bool write_out,
                          hipStream_t st, bool normed = false, const int* row_slot = nullptr) {
  const Dims& d = m->d;
  GemvArgs a{};
  a.W = m->w<int8_t>(m->P.emb_q);
  a.scale = m->w<float>(m->P.emb_s);
  a.N = d.V;
  a.K = d.d;
  a.nb = B;
  a.logits = logits;
  a.ldl = d.V;
  a.part_keys = m->ws<unsigned long long>(m->P.lm_keys);
  a.done = m->ws<unsigned int>(m->P.done);
  a.next_ids = next_ids;
  a.pos = bump_pos ? m->ws<int>(m->P.pos) : nullptr;
  a.row_slot = row_slot;
  a.out_ids = write_out ? m->ws<int>(m->P.out_ids) : nullptr;
  a.out_ld = m->lim.max_ctx;
  a.step = m->ws<int>(m->P.step);
  a.bump_step = write_out ? 1 : 0;
  a.batch0 = 0;
  if (B == 1) {
    a.x = x;
    a.ldx = d.d;
    a.x_rows = x_rows;
    a.gain = normed ? nullptr : m->w<float>(m->P.final_g);
    a.eps = m->shape.rms_eps;
    HIPCHK(launch_gemv(a, EPI_LOGITS, st));
  } else {
    bf16_t* h = m->ws<bf16_t>(m->P.h);
    if (normed) h = const_cast<bf16_t*>(x);
    else HIPCHK(launch_rmsnorm(x, rows_total, d.d, m->w<float>(m->P.final_g), m->shape.rms_eps, h, st));
    a.x = h;
    a.ldx = d.d;
    a.x_rows = x_rows;
    HIPCHK(launch_skinny(a, EPI_LOGITS, st));
  }
  return QD_OK;
}

constexpr int GEN_GRAPH_STEPS = 8;  // decode steps per captured graph in qd_generate_greedy

// ---- the kernels of one decode step, for slots 0..B-1 (rows == slots) -------------------
// work-groups per channel tile of a skinny projection: enough to cover the CUs and to
// give each of the four waves about one 128-k block, bounded by the partial buffer.
// Default policy: split only projections with fewer than 128 tiles and more than 16 rows
// (measured: below that the exchange of partials costs more than the added parallelism)
int skinny_splits(const qd_model* m, int B, int N, int K, int epi) {
  const int ctw = epi == EPI_SILU ? 2 : 1;
  const int tt = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
  const int ntiles = (N + 16 * ctw - 1) / (16 * ctw);
  const int nkb = (K + 127) / 128;
  if (m->skinny_split == 1 || (m->skinny_split == 2 && (ntiles >= 128 || tt < 2)) ||
      ntiles > SKINNY_MAX_TILES)
    return 1;
  int S = std::max((256 + ntiles - 1) / ntiles, (nkb + 3) / 4);
  S = std::min(std::min(S, nkb), SKINNY_MAX_SPLIT);
  while (S > 1 && (size_t)ntiles * S * ctw * tt * 256 > GEMM_PART_FLOATS) --S;
  return S;
}

// one projection for B rows: B == 1 runs the register GEMV (RMSNorm in its prologue when
// gain is set); B >= 2 normalizes into h first and runs the MFMA skinny GEMM
qd_status dec_proj(qd_model* m, int B, const bf16_t* x, int ldx, const float* gain,
                   const int8_t* W, const float* scale, int N, int K, int epi, bf16_t* out,
                   int ldo, hipStream_t st, int att_ns = 0) {
  GemvArgs a{};
  a.W = W; a.scale = scale; a.N = N; a.K = K; a.nb = B; a.out = out; a.ldo = ldo;
  if (B == 1) {
    a.x = x; a.ldx = ldx; a.gain = gain; a.eps = m->shape.rms_eps;
    if (att_ns > 0) {  // the row is merged from the decode attention's split partials
      a.att_po = m->ws<float>(m->P.part_o);
      a.att_ml = m->ws<float>(m->P.part_ml);
      a.att_ns = att_ns;
      a.att_D = m->d.D;
    }
    HIPCHK(launch_gemv(a, epi, st));
    return QD_OK;
  }
  a.ksplit = skinny_splits(m, B, N, K, epi);
  if (gain && m->skinny_norm && skinny_norm_ok(B, K, epi, a.ksplit)) {
    a.gain = gain;  // the RMSNorm runs inside the projection
    a.eps = m->shape.rms_eps;
  } else if (gain) {
    bf16_t* h = m->ws<bf16_t>(m->P.h);
    HIPCHK(launch_rmsnorm(x, B, K, gain, m->shape.rms_eps, h, st));
    x = h;
    ldx = K;
  }
  a.x = x; a.ldx = ldx;
  a.kpart = m->ws<float>(m->P.gemm_part);
  a.kcnt = m->ws<unsigned int>(m->P.sk_cnt);
  a.no_xstage = !m->skinny_xstage;
  HIPCHK(launch_skinny(a, epi, st));
  return QD_OK;
}

qd_status dec_qkv(qd_model* m, int l, int B, hipStream_t st) {
  const Dims& d = m->d;
  const LayerOff& o = m->P.L[l];
  return dec_proj(m, B, m->ws<bf16_t>(m->P.x), d.d, m->w<float>(o.in_g), m->w<int8_t>(o.qkv_q),
                  m->w<float>(o.qkv_s), d.NQKV, d.d, EPI_STORE, m->ws<bf16_t>(m->P.qkv), d.NQKV, st);
}

// measured on Qwen3-0.6B (8 KV heads): B = 1 at 383 positions 7.1 us (4 waves) against 7.6
// (8 waves), at ~8.2K positions 16.2 against 14.5; at ~320 positions B = 8 9.4 against 8.6,
// B = 16 10.9 against 9.2, B = 32 12.0 with 8 waves
constexpr int ATT_LONG_CTX = 2048;
int attn_waves_for(const qd_model* m, int B, int ctx) {
  if (m->attn_waves) return m->attn_waves;
  return (B * m->d.KV >= 64 || ctx > ATT_LONG_CTX) ? 8 : 4;
}

// eight waves: one work-group per CU (measured best at B x KV >= 256); four waves: as many
// as fit on a CU, at most three
int attn_occupancy_for(const qd_model* m, int B, int ctx) {
  if (m->attn_occupancy) return m->attn_occupancy;
  return attn_waves_for(m, B, ctx) == 8 ? 1 : m->attn_resident4;
}

// single-row decode with 2..ATT_DEFER_MAX_SPLITS attention splits: the splits leave their
// partials and the O projection merges them while it loads its input (QD_TUNE_ATTN_MERGE_LAST
// 1, the default); the attention's own last-split merge otherwise
bool attn_defer_merge(const qd_model* m, int B, int nsplit) {
  return B == 1 && m->attn_merge_last == 1 && nsplit >= 2 && nsplit <= ATT_DEFER_MAX_SPLITS &&
         m->d.HD <= 64 * 16 * 8;
}

qd_status dec_attn(qd_model* m, int l, int B, int nsplit, int split_len, int waves, hipStream_t st,
                   const int* row_slot = nullptr) {
  const Dims& d = m->d;
  const LayerOff& o = m->P.L[l];
  AttnDecArgs aa{};
  aa.qkv = m->ws<bf16_t>(m->P.qkv); aa.ldqkv = d.NQKV;
  aa.q_gain = m->w<float>(o.qn_g); aa.k_gain = m->w<float>(o.kn_g); aa.eps = m->shape.rms_eps;
  aa.rope = m->w<float2>(m->P.rope);
  aa.pos = m->ws<int>(m->P.pos);
  aa.row_slot = row_slot;
  aa.kcache = m->kcache(l); aa.vcache = m->vcache(l);
  aa.H = d.H; aa.KV = d.KV; aa.D = d.D; aa.max_ctx = m->lim.max_ctx; aa.B = B;
  aa.split_len = split_len; aa.nsplit = nsplit;
  aa.nwaves = waves;
  aa.merge_last = attn_defer_merge(m, B, nsplit) ? 2 : (m->attn_merge_last ? 1 : 0);
  aa.part_o = m->ws<float>(m->P.part_o); aa.part_ml = m->ws<float>(m->P.part_ml);
  aa.counters = m->ws<unsigned int>(m->P.att_cnt);
  aa.out = m->ws<bf16_t>(m->P.attn); aa.ldo = d.HD;
  HIPCHK(launch_attention_decode(aa, st));
  return QD_OK;
}

// nsplit: the attention's split count when it ran in this step (0: its output is in place)
qd_status dec_o(qd_model* m, int l, int B, hipStream_t st, int nsplit = 0) {
  const Dims& d = m->d;
  const LayerOff& o = m->P.L[l];
  return dec_proj(m, B, m->ws<bf16_t>(m->P.attn), d.HD, nullptr, m->w<int8_t>(o.o_q),
                  m->w<float>(o.o_s), d.d, d.HD, EPI_RESID, m->ws<bf16_t>(m->P.x), d.d, st,
                  attn_defer_merge(m, B, nsplit) ? nsplit : 0);
}

qd_status dec_gateup(qd_model* m, int l, int B, hipStream_t st) {
  const Dims& d = m->d;
  const LayerOff& o = m->P.L[l];
  return dec_proj(m, B, m->ws<bf16_t>(m->P.x), d.d, m->w<float>(o.post_g), m->w<int8_t>(o.gu_q),
                  m->w<float>(o.gu_s), 2 * d.I, d.d, EPI_SILU, m->ws<bf16_t>(m->P.act), d.I, st);
}

qd_status dec_down(qd_model* m, int l, int B, hipStream_t st) {
  const Dims& d = m->d;
  const LayerOff& o = m->P.L[l];
  return dec_proj(m, B, m->ws<bf16_t>(m->P.act), d.I, nullptr, m->w<int8_t>(o.dn_q),
                  m->w<float>(o.dn_s), d.d, d.I, EPI_RESID, m->ws<bf16_t>(m->P.x), d.d, st);
}

#define QDCHK(expr)                   \
  do {                                \
    qd_status s_ = (expr);            \
    if (s_ != QD_OK) return s_;       \
  } while (0)

// one decode step; positions read from the device
qd_status enqueue_decode(qd_model* m, int B, const int* in_ids, float* logits, int* next_ids,
                         bool write_out, int nsplit, int split_len, int waves, hipStream_t st,
                         const int* row_slot = nullptr) {
  const Dims& d = m->d;
  HIPCHK(launch_embed(in_ids, B, m->w<int8_t>(m->P.emb_q), m->w<float>(m->P.emb_s), d.d, d.V,
                      m->ws<bf16_t>(m->P.x), st, m->ws<int>(m->P.tok_counts), row_slot));
  for (int l = 0; l < d.L; ++l) {
    QDCHK(dec_qkv(m, l, B, st));
    QDCHK(dec_attn(m, l, B, nsplit, split_len, waves, st, row_slot));
    QDCHK(dec_o(m, l, B, st, nsplit));
    QDCHK(dec_gateup(m, l, B, st));
    QDCHK(dec_down(m, l, B, st));
  }
  return enqueue_lm_head(m, m->ws<bf16_t>(m->P.x), nullptr, B, B, logits, next_ids, true,
                         write_out, st, false, row_slot);
}

// staging layout (ints): [prompt ids: Mmax][row_slot: Mmax][row_pos: Mmax][last: B][lens: B]
// [tiles: 4 * (Mmax / FLASH_ROWS + B + 1)][pad to 8 bytes][seeds: 2B][slots: B]
size_t stage_ints(const Plan& P, int B) {
  const size_t base = (size_t)4 * P.mmax + 2 * (size_t)B + 4 * ((size_t)P.mmax / FLASH_ROWS + B + 1);
  return ((base + 1) & ~(size_t)1) + 3 * (size_t)B;
}
// the sampler's per-row seeds and a slot list (rows -> KV slots) travel to the device
// through the end of the staging area: [seeds: B x 8 bytes, 8-byte aligned][slots: B]
unsigned long long* stage_seeds(qd_model* m) {
  return reinterpret_cast<unsigned long long*>(m->hstage + m->hstage_ints - 3 * (size_t)m->lim.max_batch);
}
int* stage_slots(qd_model* m) { return m->hstage + m->hstage_ints - m->lim.max_batch; }

qd_status stage_wait(qd_model* m) {
  if (m->stage_pending) {
    HIPCHK(hipEventSynchronize(m->stage_ev));
    m->stage_pending = false;
  }
  return QD_OK;
}

qd_status stage_mark(qd_model* m, hipStream_t st) {
  HIPCHK(hipEventRecord(m->stage_ev, st));
  m->stage_pending = true;
  return QD_OK;
}

// prefill of n prompts whose ids are already in the workspace (P.ids), metadata on host
qd_status enqueue_prefill(qd_model* m, int n, const int* ids_dev, const std::vector<int>& lens,
                          float* logits, int* next_ids, bool write_out, hipStream_t st,
                          const int* slots = nullptr) {
  const Dims& d = m->d;
  const Plan& P = m->P;
  qd_status sw = stage_wait(m);
  if (sw != QD_OK) return sw;
  const int Bmax = m->lim.max_batch;
  int* h_rs = m->hstage + P.mmax;
  int* h_rp = h_rs + P.mmax;
  int* h_last = h_rp + P.mmax;
  int* h_lens = h_last + Bmax;
  int* h_tiles = h_lens + Bmax;
  // attention query tiles of 128 rows when they alone give every CU two work-groups (head
  // dims up to 128), else 64
  int tile_rows = m->flash_rows;
  if (tile_rows == 0) {
    long long t128 = 0;
    for (int b = 0; b < n; ++b) t128 += (lens[b] + 2 * FLASH_ROWS - 1) / (2 * FLASH_ROWS);
    tile_rows = (d.D <= 128 && t128 * d.H >= 512) ? 2 * FLASH_ROWS : FLASH_ROWS;
  }
  if (d.D > 128) tile_rows = FLASH_ROWS;
  int M = 0, n_tiles = 0;
  for (int b = 0; b < n; ++b) {
    for (int p0 = 0; p0 < lens[b]; p0 += tile_rows) {
      h_tiles[4 * n_tiles + 0] = M + p0;
      h_tiles[4 * n_tiles + 1] = slots ? slots[b] : b;
      h_tiles[4 * n_tiles + 2] = p0;
      h_tiles[4 * n_tiles + 3] = std::min(tile_rows, lens[b] - p0);
      ++n_tiles;
    }
    for (int t = 0; t < lens[b]; ++t) {
      h_rs[M + t] = slots ? slots[b] : b;
      h_rp[M + t] = t;
    }
    M += lens[b];
    h_last[b] = M - 1;
    h_lens[b] = lens[b];
  }
  int* row_slot = m->ws<int>(P.row_slot);
  int* row_pos = m->ws<int>(P.row_pos);
  int* last_rows = m->ws<int>(P.last_rows);
  int* dlens = m->ws<int>(P.lens);
  int4* dtiles = m->ws<int4>(P.tiles);
  HIPCHK(hipMemcpyAsync(row_slot, h_rs, M * 4, hipMemcpyHostToDevice, st));
  HIPCHK(hipMemcpyAsync(row_pos, h_rp, M * 4, hipMemcpyHostToDevice, st));
  HIPCHK(hipMemcpyAsync(last_rows, h_last, n * 4, hipMemcpyHostToDevice, st));
  HIPCHK(hipMemcpyAsync(dlens, h_lens, n * 4, hipMemcpyHostToDevice, st));
  HIPCHK(hipMemcpyAsync(dtiles, h_tiles, (size_t)n_tiles * 16, hipMemcpyHostToDevice, st));
  int* dslots = nullptr;
  if (slots) {
    int* hs = stage_slots(m);
    std::memcpy(hs, slots, (size_t)n * 4);
    dslots = m->ws<int>(P.slot_map);
    HIPCHK(hipMemcpyAsync(dslots, hs, (size_t)n * 4, hipMemcpyHostToDevice, st));
  }
  sw = stage_mark(m, st);
  if (sw != QD_OK) return sw;

  bf16_t* x = m->ws<bf16_t>(P.x);
  bf16_t* h = m->ws<bf16_t>(P.h);
  bf16_t* qkv = m->ws<bf16_t>(P.qkv);
  bf16_t* attn = m->ws<bf16_t>(P.attn);
  bf16_t* act = m->ws<bf16_t>(P.act);
  float* gpart = m->ws<float>(P.gemm_part);
  // the sampler's token counts and draw numbers restart with each prompt; the embedding
  // counts the prompt tokens
  HIPCHK(launch_reset_seq(m->ws<int>(P.tok_counts), m->ws<int>(P.draws), dslots, n, d.V, st));
  HIPCHK(launch_embed(ids_dev, M, m->w<int8_t>(P.emb_q), m->w<float>(P.emb_s), d.d, d.V, x, st,
                      m->ws<int>(P.tok_counts), row_slot));
  // the input RMSNorm of layer 0; every later one (and the final norm) runs fused with
  // the split-K merge of the down projection before it
  HIPCHK(launch_rmsnorm(x, M, d.d, m->w<float>(P.L[0].in_g), m->shape.rms_eps, h, st));
  // residual projection (O or down) with deferred split-K, then x's RMSNorm with gain ng
  auto resid_proj = [&](GemmArgs g, const float* ng) -> hipError_t {
    g.defer = 1;
    int so = 1;
    hipError_t e = launch_gemm(g, st, &so);
    if (e != hipSuccess) return e;
    if (so > 1) return launch_resid_norm(x, M, d.d, gpart, so, g.scale, ng, m->shape.rms_eps, h, st);
    return launch_rmsnorm(x, M, d.d, ng, m->shape.rms_eps, h, st);
  };
  for (int l = 0; l < d.L; ++l) {
    const LayerOff& o = P.L[l];
    GemmArgs g{};
    g.A = h; g.lda = d.d; g.W = m->w<int8_t>(o.qkv_q); g.scale = m->w<float>(o.qkv_s);
    g.M = M; g.N = d.NQKV; g.K = d.d; g.epi = EPI_STORE; g.out = qkv; g.ldo = d.NQKV; g.part = gpart; g.cnt = m->ws<unsigned int>(P.sk_cnt); g.splits = m->gemm_splits; g.use_ks = m->gemm_ks;
    RopeArgs ra{};
    ra.qkv = qkv; ra.ldqkv = d.NQKV;
    ra.q_gain = m->w<float>(o.qn_g); ra.k_gain = m->w<float>(o.kn_g); ra.eps = m->shape.rms_eps;
    ra.rope = m->w<float2>(P.rope);
    ra.row_slot = row_slot; ra.row_pos = row_pos;
    ra.kcache = m->kcache(l); ra.vcache = m->vcache(l);
    ra.H = d.H; ra.KV = d.KV; ra.D = d.D; ra.max_ctx = m->lim.max_ctx; ra.M = M;
    g.fuse_rope = m->gemm_rope; g.rope = ra;
    int rope_done = 0;
    HIPCHK(launch_gemm(g, st, nullptr, &rope_done));
    if (!rope_done) HIPCHK(launch_qk_rope(ra, st));
    FlashArgs fa{};
    fa.q = qkv; fa.ldq = d.NQKV;
    fa.kcache = m->kcache(l); fa.vcache = m->vcache(l);
    fa.tiles = dtiles;
    fa.H = d.H; fa.KV = d.KV; fa.D = d.D; fa.max_ctx = m->lim.max_ctx;
    fa.out = attn; fa.ldo = d.HD;
    HIPCHK(launch_flash_prefill(fa, n_tiles, tile_rows, st));
    g = GemmArgs{};
    g.A = attn; g.lda = d.HD; g.W = m->w<int8_t>(o.o_q); g.scale = m->w<float>(o.o_s);
    g.M = M; g.N = d.d; g.K = d.HD; g.epi = EPI_RESID; g.out = x; g.ldo = d.d; g.part = gpart; g.cnt = m->ws<unsigned int>(P.sk_cnt); g.splits = m->gemm_splits; g.use_ks = m->gemm_ks;
    HIPCHK(resid_proj(g, m->w<float>(o.post_g)));
    g = GemmArgs{};
    g.A = h; g.lda = d.d; g.W = m->w<int8_t>(o.gu_q); g.scale = m->w<float>(o.gu_s);
    g.M = M; g.N = 2 * d.I; g.K = d.d; g.epi = EPI_SILU; g.out = act; g.ldo = d.I; g.part = gpart; g.cnt = m->ws<unsigned int>(P.sk_cnt); g.splits = m->gemm_splits; g.use_ks = m->gemm_ks;
    HIPCHK(launch_gemm(g, st));
    g = GemmArgs{};
    g.A = act; g.lda = d.I; g.W = m->w<int8_t>(o.dn_q); g.scale = m->w<float>(o.dn_s);
    g.M = M; g.N = d.d; g.K = d.I; g.epi = EPI_RESID; g.out = x; g.ldo = d.d; g.part = gpart; g.cnt = m->ws<unsigned int>(P.sk_cnt); g.splits = m->gemm_splits; g.use_ks = m->gemm_ks;
    HIPCHK(resid_proj(g, l + 1 < d.L ? m->w<float>(P.L[l + 1].in_g) : m->w<float>(P.final_g)));
  }
  // h holds the final-normalized rows
  qd_status s = enqueue_lm_head(m, h, last_rows, M, n, logits, next_ids, false, write_out, st, true);
  if (s != QD_OK) return s;
  HIPCHK(launch_set_positions(m->ws<int>(P.pos), dlens, dslots, n, st));
  return QD_OK;
}

std::string check_ids(const int32_t* ids, long n, int V) {
  for (long i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= V)
      return "token id " + std::to_string(ids[i]) + " at index " + std::to_string(i) +
             " is outside [0, " + std::to_string(V) + ")";
  return "";
}

}  // namespace

// ============================================================================================
extern "C" {

const char* qd_last_error(void) { return g_err.c_str(); }

qd_status qd_check_shape(const qd_model_shape* shape) {
  g_err.clear();
  const std::string p = gate_problems(shape);
  if (!p.empty()) return fail(QD_ERR_UNSUPPORTED_ARCH, "unsupported architecture: " + p);
  return QD_OK;
}

qd_status qd_query_sizes(const qd_model_shape* shape, const qd_limits* limits, qd_sizes* out) {
  qd_status st = qd_check_shape(shape);
  if (st != QD_OK) return st;
  if ((st = check_limits(limits)) != QD_OK) return st;
  if (!out) return fail(QD_ERR_INVALID_ARGUMENTS, "out is NULL");
  const std::string pb = prefill_bound_problem(*shape, *limits);
  if (!pb.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, pb);
  const Plan P = make_plan(*shape, *limits);
  out->weight_bytes = P.weight_bytes;
  out->kv_bytes = P.kv_bytes;
  out->workspace_bytes = P.ws_bytes;
  out->packed_model_bytes = P.packed;
  return QD_OK;
}

namespace {
// checks the limits and caller buffers and creates the handle (no GPU work)
qd_status open_model(const qd_model_shape* shape, const qd_limits* limits,
                     const qd_buffers* bufs, qd_model** out, hipDeviceProp_t* prop) {
  const std::string pb = prefill_bound_problem(*shape, *limits);
  if (!pb.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, pb);
  const Plan P = make_plan(*shape, *limits);
  if (!bufs || !bufs->weights || !bufs->kv || !bufs->workspace)
    return fail(QD_ERR_INVALID_ARGUMENTS, "a device buffer pointer is NULL");
  std::string small;
  if (bufs->weight_bytes < P.weight_bytes)
    small += "weights " + std::to_string(bufs->weight_bytes) + " < " + std::to_string(P.weight_bytes) + "; ";
  if (bufs->kv_bytes < P.kv_bytes)
    small += "kv " + std::to_string(bufs->kv_bytes) + " < " + std::to_string(P.kv_bytes) + "; ";
  if (bufs->workspace_bytes < P.ws_bytes)
    small += "workspace " + std::to_string(bufs->workspace_bytes) + " < " + std::to_string(P.ws_bytes) + "; ";
  if (!small.empty()) return fail(QD_ERR_BUFFER_TOO_SMALL, "buffers too small: " + small);
  if ((((uintptr_t)bufs->weights) | ((uintptr_t)bufs->kv) | ((uintptr_t)bufs->workspace)) & 255)
    return fail(QD_ERR_INVALID_ARGUMENTS, "device buffers must be 256-byte aligned");
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  HIPCHK(hipGetDeviceProperties(prop, dev));
  if (std::strncmp(prop->gcnArchName, "gfx950", 6) != 0)
    return fail(QD_ERR_DEVICE, std::string("device is ") + prop->gcnArchName + ", need gfx950");
  qd_model* m = new qd_model();
  m->shape = *shape;
  m->lim = *limits;
  m->d = dims_of(*shape);
  m->P = P;
  m->W = (char*)bufs->weights;
  m->KVb = (char*)bufs->kv;
  m->WS = (char*)bufs->workspace;
  m->device = dev;
  m->host_pos.assign(limits->max_batch, 0);
  *out = m;
  return QD_OK;
}

// everything after the weights are in place: RoPE table, device state, streams, staging
qd_status finish_model(qd_model* m, const hipDeviceProp_t& prop, hipStream_t s) {
  const Plan& P = m->P;
  const Dims& d = m->d;
  HIPCHK(launch_rope_table(m->w<float2>(P.rope), m->lim.max_ctx, d.D, m->shape.rope_theta, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.pos), m->lim.max_batch, 0, s));
  HIPCHK(launch_iota(m->ws<int>(P.slot_ident), m->lim.max_batch, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.att_cnt), m->lim.max_batch * d.KV, 0, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.sk_cnt), SKINNY_MAX_TILES, 0, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.done), 16, 0, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.step), 16, 0, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.smp_rowmax), m->lim.max_batch, 0, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.smp_hist), m->lim.max_batch * 256, 0, s));
  HIPCHK(launch_fill_i32(m->ws<int>(P.smp_ncand), m->lim.max_batch, 0, s));
  HIPCHK(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking));
  m->hstage_ints = stage_ints(P, m->lim.max_batch);
  HIPCHK(hipHostMalloc((void**)&m->hstage, m->hstage_ints * 4, hipHostMallocDefault));
  HIPCHK(hipEventCreateWithFlags(&m->stage_ev, hipEventDisableTiming));
  for (int i = 0; i < 3; ++i) HIPCHK(hipEventCreate(&m->ev[i]));
  HIPCHK(hipStreamSynchronize(s));
  // the fixed scratch of qd_sample_noalloc: its address on this device, looked up once here
  HIPCHK(sample_scratch_address(&m->noalloc_scratch));
  int res4 = 0;  // shapes the decode attention kernel does not take keep the default
  if (attention_decode_residency(m->d.D, m->d.G, 4, &res4) == hipSuccess && res4 > 0)
    m->attn_resident4 = std::min(3, res4);
  return QD_OK;
}

// the quantized regions of the weights arena, in cache order: (offset, bytes)
std::vector<std::pair<size_t, size_t>> cache_regions(const qd_model* m) {
  const Plan& P = m->P;
  const Dims& d = m->d;
  std::vector<std::pair<size_t, size_t>> r;
  r.push_back({P.emb_q, (size_t)d.V * d.d});
  r.push_back({P.emb_s, (size_t)d.V * 4});
  r.push_back({P.final_g, (size_t)d.d * 4});
  for (int l = 0; l < d.L; ++l) {
    const LayerOff& o = P.L[l];
    r.push_back({o.qkv_q, (size_t)d.NQKV * d.d});
    r.push_back({o.qkv_s, (size_t)d.NQKV * 4});
    r.push_back({o.o_q, (size_t)d.d * d.HD});
    r.push_back({o.o_s, (size_t)d.d * 4});
    r.push_back({o.gu_q, (size_t)2 * d.I * d.d});
    r.push_back({o.gu_s, (size_t)2 * d.I * 4});
    r.push_back({o.dn_q, (size_t)d.d * d.I});
    r.push_back({o.dn_s, (size_t)d.d * 4});
    r.push_back({o.in_g, (size_t)d.d * 4});
    r.push_back({o.post_g, (size_t)d.d * 4});
    r.push_back({o.qn_g, (size_t)d.D * 4});
    r.push_back({o.kn_g, (size_t)d.D * 4});
  }
  return r;
}

CacheHeader cache_header_for(const qd_model_shape& s, const uint8_t digest[32], uint64_t payload) {
  CacheHeader h;
  std::memset(&h, 0, sizeof(h));
  std::memcpy(h.magic, "QDI8WCV1", 8);
  h.version = 2;
  h.header_bytes = sizeof(CacheHeader);
  const int32_t v[7] = {s.hidden, s.n_layers, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab};
  for (int i = 0; i < 7; ++i) h.dims[i] = (uint32_t)v[i];
  std::memcpy(&h.dims[7], &s.rms_eps, 4);
  std::memcpy(&h.dims[8], &s.rope_theta, 4);
  std::memcpy(h.source_digest, digest, 32);
  h.payload_bytes = payload;
  return h;
}
}  // namespace

qd_status qd_load_weights(const qd_model_shape* shape, const qd_limits* limits,
                          const qd_weights_f32* wts, const qd_buffers* bufs, qd_stream stream,
                          qd_model** out) {
  qd_status st = qd_check_shape(shape);
  if (st != QD_OK) return st;
  if ((st = check_limits(limits)) != QD_OK) return st;
  if (!out) return fail(QD_ERR_INVALID_ARGUMENTS, "out is NULL");
  *out = nullptr;
  // every tensor must be present ("checkpoint_not_found" names each missing one)
  std::string missing;
  auto need = [&](const void* p, const std::string& n) {
    if (!p) missing += (missing.empty() ? "" : ", ") + n;
  };
  if (!wts) return fail(QD_ERR_CHECKPOINT_NOT_FOUND, "weights is NULL");
  need(wts->embed, "embed_tokens");
  need(wts->final_norm, "norm");
  if (!wts->layers) {
    missing += (missing.empty() ? "" : ", ") + std::string("layers");
  } else {
    for (int l = 0; l < shape->n_layers; ++l) {
      const qd_layer_f32& L = wts->layers[l];
      const std::string pre = "layers." + std::to_string(l) + ".";
      need(L.q, pre + "q_proj"); need(L.k, pre + "k_proj"); need(L.v, pre + "v_proj");
      need(L.o, pre + "o_proj"); need(L.gate, pre + "gate_proj"); need(L.up, pre + "up_proj");
      need(L.down, pre + "down_proj"); need(L.in_norm, pre + "input_layernorm");
      need(L.post_norm, pre + "post_attention_layernorm"); need(L.q_norm, pre + "q_norm");
      need(L.k_norm, pre + "k_norm");
    }
  }
  if (!missing.empty()) return fail(QD_ERR_CHECKPOINT_NOT_FOUND, "missing tensors: " + missing);
  hipDeviceProp_t prop;
  qd_model* m = nullptr;
  QDCHK(open_model(shape, limits, bufs, &m, &prop));
  const Plan& P = m->P;
  hipStream_t s = (hipStream_t)stream;
  auto cleanup_fail = [&](qd_status code) {
    qd_free(m);
    return code;
  };
#define LCHK(expr)                                                                        \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return cleanup_fail(fail(QD_ERR_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_))); \
  } while (0)
  const Dims& d = m->d;
  LCHK(launch_quantize_rows(wts->embed, d.V, d.d, m->w<int8_t>(P.emb_q), m->w<float>(P.emb_s), 0, -1, s));
  LCHK(hipMemcpyAsync(m->w<float>(P.final_g), wts->final_norm, d.d * 4, hipMemcpyDeviceToDevice, s));
  for (int l = 0; l < d.L; ++l) {
    const qd_layer_f32& L = wts->layers[l];
    const LayerOff& o = P.L[l];
    int8_t* qkv = m->w<int8_t>(o.qkv_q);
    float* qkvs = m->w<float>(o.qkv_s);
    LCHK(launch_quantize_rows(L.q, d.HD, d.d, qkv, qkvs, 0, -1, s));
    LCHK(launch_quantize_rows(L.k, d.KVD, d.d, qkv, qkvs, d.HD, -1, s));
    LCHK(launch_quantize_rows(L.v, d.KVD, d.d, qkv, qkvs, d.HD + d.KVD, -1, s));
    LCHK(launch_quantize_rows(L.o, d.d, d.HD, m->w<int8_t>(o.o_q), m->w<float>(o.o_s), 0, -1, s));
    LCHK(launch_quantize_rows(L.gate, d.I, d.d, m->w<int8_t>(o.gu_q), m->w<float>(o.gu_s), 0, 0, s));
    LCHK(launch_quantize_rows(L.up, d.I, d.d, m->w<int8_t>(o.gu_q), m->w<float>(o.gu_s), 0, 1, s));
    LCHK(launch_quantize_rows(L.down, d.d, d.I, m->w<int8_t>(o.dn_q), m->w<float>(o.dn_s), 0, -1, s));
    LCHK(hipMemcpyAsync(m->w<float>(o.in_g), L.in_norm, d.d * 4, hipMemcpyDeviceToDevice, s));
    LCHK(hipMemcpyAsync(m->w<float>(o.post_g), L.post_norm, d.d * 4, hipMemcpyDeviceToDevice, s));
    LCHK(hipMemcpyAsync(m->w<float>(o.qn_g), L.q_norm, d.D * 4, hipMemcpyDeviceToDevice, s));
    LCHK(hipMemcpyAsync(m->w<float>(o.kn_g), L.k_norm, d.D * 4, hipMemcpyDeviceToDevice, s));
  }
#undef LCHK
  st = finish_model(m, prop, s);
  if (st != QD_OK) return cleanup_fail(st);
  *out = m;
  return QD_OK;
}

qd_status qd_save_cache(qd_model* m, const char* path, const uint8_t* source_digest,
                        qd_stream stream) {
  g_err.clear();
  if (!m || !path || !source_digest) return fail(QD_ERR_INVALID_ARGUMENTS, "NULL argument");
  HIPCHK(hipStreamSynchronize((hipStream_t)stream));
  const auto regions = cache_regions(m);
  uint64_t total = 0;
  for (const auto& r : regions) total += r.second;
  std::vector<uint8_t> payload(total);
  uint64_t at = 0;
  for (const auto& r : regions) {
    HIPCHK(hipMemcpy(payload.data() + at, m->W + r.first, r.second, hipMemcpyDeviceToHost));
    at += r.second;
  }
  CacheHeader h = cache_header_for(m->shape, source_digest, total);
  chunked_sha256(payload.data(), payload.size(), h.payload_sha256);
  const std::string tmp = std::string(path) + ".tmp";
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) return fail(QD_ERR_INVALID_ARGUMENTS, "cannot write " + tmp);
  const bool ok = std::fwrite(&h, sizeof(h), 1, f) == 1 &&
                  std::fwrite(payload.data(), 1, payload.size(), f) == payload.size();
  const bool closed = std::fclose(f) == 0;
  if (!ok || !closed || std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return fail(QD_ERR_INVALID_ARGUMENTS, std::string("writing the cache ") + path + " failed");
  }
  return QD_OK;
}

namespace {
// reads and gates a cache file against a shape and source digest; payload out on success
qd_status read_cache(const qd_model_shape* shape, const char* path, const uint8_t* digest,
                     uint64_t expect_payload, std::vector<uint8_t>* payload) {
  FILE* f = std::fopen(path, "rb");
  if (!f) return fail(QD_ERR_CACHE_MISS, std::string("no cache at ") + path);
  CacheHeader h;
  std::memset(&h, 0, sizeof(h));
  const size_t got = std::fread(&h, 1, sizeof(h), f);
  std::string p;
  if (got != sizeof(h)) p = "file shorter than the header";
  else p = cache_header_problems(h, cache_header_for(*shape, digest, expect_payload));
  if (p.empty()) {
    std::fseek(f, 0, SEEK_END);
    const long len = std::ftell(f);
    if (len < 0 || (uint64_t)len != sizeof(h) + expect_payload)
      p = "file length " + std::to_string(len) + " != " + std::to_string(sizeof(h) + expect_payload);
  }
  if (p.empty()) {
    payload->resize(expect_payload);
    std::fseek(f, (long)sizeof(h), SEEK_SET);
    if (std::fread(payload->data(), 1, expect_payload, f) != expect_payload) p = "short read";
  }
  std::fclose(f);
  if (p.empty()) {
    uint8_t sum[32];
    chunked_sha256(payload->data(), payload->size(), sum);
    if (std::memcmp(sum, h.payload_sha256, 32) != 0) p = "payload digest (chunked SHA-256) differs";
  }
  if (!p.empty()) return fail(QD_ERR_CACHE_MISS, std::string(path) + ": " + p);
  return QD_OK;
}
}  // namespace

qd_status qd_check_cache(const qd_model_shape* shape, const char* path, const uint8_t* source_digest) {
  g_err.clear();
  qd_status st = qd_check_shape(shape);
  if (st != QD_OK) return st;
  if (!path || !source_digest) return fail(QD_ERR_INVALID_ARGUMENTS, "NULL argument");
  const qd_limits lim{1, 64, 64};
  qd_model tmp;
  tmp.shape = *shape;
  tmp.d = dims_of(*shape);
  tmp.P = make_plan(*shape, lim);
  uint64_t total = 0;
  for (const auto& r : cache_regions(&tmp)) total += r.second;
  std::vector<uint8_t> payload;
  return read_cache(shape, path, source_digest, total, &payload);
}

qd_status qd_load_cache(const qd_model_shape* shape, const qd_limits* limits, const char* path,
                        const uint8_t* source_digest, const qd_buffers* bufs, qd_stream stream,
                        qd_model** out) {
  g_err.clear();
  qd_status st = qd_check_shape(shape);
  if (st != QD_OK) return st;
  if ((st = check_limits(limits)) != QD_OK) return st;
  if (!out || !path || !source_digest) return fail(QD_ERR_INVALID_ARGUMENTS, "NULL argument");
  *out = nullptr;
  hipDeviceProp_t prop;
  qd_model* m = nullptr;
  QDCHK(open_model(shape, limits, bufs, &m, &prop));
  const auto regions = cache_regions(m);
  uint64_t total = 0;
  for (const auto& r : regions) total += r.second;
  std::vector<uint8_t> payload;
  st = read_cache(shape, path, source_digest, total, &payload);
  if (st != QD_OK) {
    const std::string msg = g_err;
    qd_free(m);
    g_err = msg;
    return st;
  }
  hipStream_t s = (hipStream_t)stream;
  uint64_t at = 0;
  for (const auto& r : regions) {
    const hipError_t e = hipMemcpy(m->W + r.first, payload.data() + at, r.second, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      qd_free(m);
      return fail(QD_ERR_DEVICE, std::string("hipMemcpy: ") + hipGetErrorString(e));
    }
    at += r.second;
  }
  st = finish_model(m, prop, s);
  if (st != QD_OK) {
    qd_free(m);
    return st;
  }
  *out = m;
  return QD_OK;
}

qd_status qd_sha256(const void* data, uint64_t n, uint8_t* out32) {
  g_err.clear();
  if ((!data && n) || !out32) return fail(QD_ERR_INVALID_ARGUMENTS, "NULL argument");
  Sha256 sha;
  sha.update(data, (size_t)n);
  sha.final(out32);
  return QD_OK;
}

qd_status qd_export_quantized(qd_model* m, int32_t tensor, int32_t layer, int8_t* codes_host,
                              float* scales_host, qd_stream stream) {
  g_err.clear();
  if (!m || !codes_host || !scales_host) return fail(QD_ERR_INVALID_ARGUMENTS, "NULL argument");
  const Dims& d = m->d;
  if (tensor != QD_T_EMBED && (layer < 0 || layer >= d.L))
    return fail(QD_ERR_INVALID_ARGUMENTS, "layer out of range");
  hipStream_t s = (hipStream_t)stream;
  const int8_t* q = nullptr;
  const float* sc = nullptr;
  int rows = 0, cols = 0, row0 = 0, half = -1;
  const LayerOff* o = tensor == QD_T_EMBED ? nullptr : &m->P.L[layer];
  switch (tensor) {
    case QD_T_EMBED: q = m->w<int8_t>(m->P.emb_q); sc = m->w<float>(m->P.emb_s); rows = d.V; cols = d.d; break;
    case QD_T_Q: q = m->w<int8_t>(o->qkv_q); sc = m->w<float>(o->qkv_s); rows = d.HD; cols = d.d; break;
    case QD_T_K: q = m->w<int8_t>(o->qkv_q); sc = m->w<float>(o->qkv_s); rows = d.KVD; cols = d.d; row0 = d.HD; break;
    case QD_T_V: q = m->w<int8_t>(o->qkv_q); sc = m->w<float>(o->qkv_s); rows = d.KVD; cols = d.d; row0 = d.HD + d.KVD; break;
    case QD_T_O: q = m->w<int8_t>(o->o_q); sc = m->w<float>(o->o_s); rows = d.d; cols = d.HD; break;
    case QD_T_GATE: q = m->w<int8_t>(o->gu_q); sc = m->w<float>(o->gu_s); rows = d.I; cols = d.d; half = 0; break;
    case QD_T_UP: q = m->w<int8_t>(o->gu_q); sc = m->w<float>(o->gu_s); rows = d.I; cols = d.d; half = 1; break;
    case QD_T_DOWN: q = m->w<int8_t>(o->dn_q); sc = m->w<float>(o->dn_s); rows = d.d; cols = d.I; break;
    default: return fail(QD_ERR_INVALID_ARGUMENTS, "unknown tensor id");
  }
  if (half < 0) {
    HIPCHK(hipMemcpyAsync(codes_host, q + (size_t)row0 * cols, (size_t)rows * cols, hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(scales_host, sc + row0, (size_t)rows * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
  } else {
    std::vector<int8_t> tq((size_t)2 * rows * cols);
    std::vector<float> ts((size_t)2 * rows);
    HIPCHK(hipMemcpyAsync(tq.data(), q, tq.size(), hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(ts.data(), sc, ts.size() * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    for (int j = 0; j < rows; ++j) {
      const int r = gu_row(j, half);
      std::memcpy(codes_host + (size_t)j * cols, tq.data() + (size_t)r * cols, cols);
      scales_host[j] = ts[r];
    }
  }
  return QD_OK;
}

namespace {
// a host slot list: n distinct slots in [0, max_batch); "" when valid
std::string check_slots(const qd_model* m, int n, const int32_t* slots) {
  std::vector<char> seen(m->lim.max_batch, 0);
  for (int b = 0; b < n; ++b) {
    const int sl = slots[b];
    if (sl < 0 || sl >= m->lim.max_batch)
      return "slot " + std::to_string(sl) + " of row " + std::to_string(b) + " is outside [0, max_batch)";
    if (seen[sl]) return "slot " + std::to_string(sl) + " is listed twice";
    seen[sl] = 1;
  }
  return "";
}

qd_status prefill_impl(qd_model* m, int32_t n_seqs, const int32_t* slots, const int32_t* ids_dev,
                       const int32_t* ids_host, const int32_t* lens_host, float* logits_dev,
                       int32_t* next_ids_dev, qd_stream stream) {
  g_err.clear();
  if (!m) return fail(QD_ERR_INVALID_ARGUMENTS, "model is NULL");
  if (n_seqs < 1 || n_seqs > m->lim.max_batch)
    return fail(QD_ERR_INVALID_ARGUMENTS, "n_seqs must be in [1, max_batch]");
  if (!ids_dev || !lens_host || !next_ids_dev)
    return fail(QD_ERR_INVALID_ARGUMENTS, "ids_dev, lens_host and next_ids_dev must be set");
  if (slots) {
    const std::string e = check_slots(m, n_seqs, slots);
    if (!e.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, e);
  }
  std::vector<int> lens(lens_host, lens_host + n_seqs);
  long total = 0;
  for (int b = 0; b < n_seqs; ++b) {
    if (lens[b] < 1) return fail(QD_ERR_INVALID_ARGUMENTS, "empty prompt for sequence " + std::to_string(b));
    if (lens[b] > m->lim.max_ctx)
      return fail(QD_ERR_INVALID_ARGUMENTS, "prompt of sequence " + std::to_string(b) + " exceeds max_ctx");
    total += lens[b];
  }
  if (total > m->lim.max_prefill_tokens)
    return fail(QD_ERR_INVALID_ARGUMENTS, "prompt tokens exceed max_prefill_tokens");
  if (ids_host) {
    const std::string e = check_ids(ids_host, total, m->d.V);
    if (!e.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, e);
  }
  qd_status s = enqueue_prefill(m, n_seqs, ids_dev, lens, logits_dev, next_ids_dev, false,
                                (hipStream_t)stream, slots);
  if (s == QD_OK)
    for (int b = 0; b < n_seqs; ++b) m->host_pos[slots ? slots[b] : b] = lens[b];
  return s;
}

qd_status decode_impl(qd_model* m, int32_t B, const int32_t* slots, const int32_t* in_ids_dev,
                      float* logits_dev, int32_t* next_ids_dev, qd_stream stream) {
  g_err.clear();
  if (!m) return fail(QD_ERR_INVALID_ARGUMENTS, "model is NULL");
  if (B < 1 || B > m->lim.max_batch) return fail(QD_ERR_INVALID_ARGUMENTS, "B must be in [1, max_batch]");
  if (!in_ids_dev || !next_ids_dev) return fail(QD_ERR_INVALID_ARGUMENTS, "ids pointers must be set");
  if (slots) {
    const std::string e = check_slots(m, B, slots);
    if (!e.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, e);
  }
  int ctx = 0;
  for (int b = 0; b < B; ++b) {
    const int sl = slots ? slots[b] : b;
    if (slots && m->host_pos[sl] < 1)
      return fail(QD_ERR_INVALID_ARGUMENTS, "slot " + std::to_string(sl) + " holds no prompt");
    if (m->host_pos[sl] >= m->lim.max_ctx)
      return fail(QD_ERR_INVALID_ARGUMENTS, "slot " + std::to_string(sl) + " is full (max_ctx)");
    ctx = std::max(ctx, m->host_pos[sl] + 1);
  }
  hipStream_t st = (hipStream_t)stream;
  qd_status s;
  {
    const int* row_slot = nullptr;
    if (slots) {
      QDCHK(stage_wait(m));
      int* hs = stage_slots(m);
      std::memcpy(hs, slots, (size_t)B * 4);
      int* ds = m->ws<int>(m->P.slot_map);
      HIPCHK(hipMemcpyAsync(ds, hs, (size_t)B * 4, hipMemcpyHostToDevice, st));
      QDCHK(stage_mark(m, st));
      row_slot = ds;
    }
    int nsplit, split_len;
    attn_split(ctx, m->P.nsplit_cap, m->attn_max_splits, m->attn_min_chunks, attn_occupancy_for(m, B, ctx), B * m->d.KV, &nsplit,
               &split_len);
    s = enqueue_decode(m, B, in_ids_dev, logits_dev, next_ids_dev, false, nsplit, split_len,
                       attn_waves_for(m, B, ctx), st, row_slot);
  }
  if (s == QD_OK)
    for (int b = 0; b < B; ++b) m->host_pos[slots ? slots[b] : b] += 1;
  return s;
}
}  // namespace

qd_status qd_prefill(qd_model* m, int32_t n_seqs, const int32_t* ids_dev, const int32_t* ids_host,
                     const int32_t* lens_host, float* logits_dev, int32_t* next_ids_dev,
                     qd_stream stream) {
  return prefill_impl(m, n_seqs, nullptr, ids_dev, ids_host, lens_host, logits_dev, next_ids_dev,
                      stream);
}

qd_status qd_prefill_slots(qd_model* m, int32_t n_seqs, const int32_t* slots_host,
                           const int32_t* ids_dev, const int32_t* ids_host,
                           const int32_t* lens_host, float* logits_dev, int32_t* next_ids_dev,
                           qd_stream stream) {
  if (!slots_host) {
    g_err.clear();
    return fail(QD_ERR_INVALID_ARGUMENTS, "slots_host must be set");
  }
  return prefill_impl(m, n_seqs, slots_host, ids_dev, ids_host, lens_host, logits_dev,
                      next_ids_dev, stream);
}

qd_status qd_decode_step(qd_model* m, int32_t B, const int32_t* in_ids_dev, float* logits_dev,
                         int32_t* next_ids_dev, qd_stream stream) {
  return decode_impl(m, B, nullptr, in_ids_dev, logits_dev, next_ids_dev, stream);
}

qd_status qd_decode_step_slots(qd_model* m, int32_t B, const int32_t* slots_host,
                               const int32_t* in_ids_dev, float* logits_dev,
                               int32_t* next_ids_dev, qd_stream stream) {
  if (!slots_host) {
    g_err.clear();
    return fail(QD_ERR_INVALID_ARGUMENTS, "slots_host must be set");
  }
  return decode_impl(m, B, slots_host, in_ids_dev, logits_dev, next_ids_dev, stream);
}

namespace {
// qd_sample and qd_sample_noalloc: the same checks and kernels; noalloc takes the per-call
// scratch (penalized rows, histograms, candidates, counters, staged seeds and slots) from
// the fixed device array instead of the model's workspace
qd_status sample_impl(qd_model* m, int32_t B, const int32_t* slots_host, const qd_sampling* params,
                      const uint64_t* seeds_host, const float* logits_dev, int32_t* next_ids_dev,
                      qd_stream stream, bool noalloc) {
  g_err.clear();
  if (!m) return fail(QD_ERR_INVALID_ARGUMENTS, "model is NULL");
  if (B < 1 || B > m->lim.max_batch) return fail(QD_ERR_INVALID_ARGUMENTS, "B must be in [1, max_batch]");
  if (noalloc && (B > NOALLOC_MAX_ROWS || (size_t)B * (size_t)m->d.V > NOALLOC_Z_FLOATS))
    return fail(QD_ERR_INVALID_ARGUMENTS,
                "qd_sample_noalloc takes at most " + std::to_string(NOALLOC_MAX_ROWS) +
                    " rows and rows x vocab <= " + std::to_string(NOALLOC_Z_FLOATS) +
                    " (its fixed scratch); got " + std::to_string(B) + " rows x " +
                    std::to_string(m->d.V));
  if (!params || !seeds_host || !logits_dev || !next_ids_dev)
    return fail(QD_ERR_INVALID_ARGUMENTS, "params, seeds_host, logits_dev and next_ids_dev must be set");
  std::string p;
  const qd_sampling& q = *params;
  if (!(q.temperature > 0.0f) || !std::isfinite(q.temperature)) p += "temperature must be > 0; ";
  if (q.top_k < 1 || q.top_k > SMP_MAXK) p += "top_k must be in [1, " + std::to_string(SMP_MAXK) + "]; ";
  if (!(q.min_p >= 0.0f && q.min_p <= 1.0f)) p += "min_p must be in [0, 1]; ";
  if (!(q.top_p > 0.0f && q.top_p <= 1.0f)) p += "top_p must be in (0, 1]; ";
  if (!(q.repeat_penalty > 0.0f) || !std::isfinite(q.repeat_penalty)) p += "repeat_penalty must be > 0; ";
  if (!std::isfinite(q.presence_penalty) || !std::isfinite(q.frequency_penalty)) p += "penalties must be finite; ";
  if (slots_host) {
    const std::string e = check_slots(m, B, slots_host);
    if (!e.empty()) p += e + "; ";
  }
  for (int b = 0; b < B && p.empty(); ++b) {
    const int sl = slots_host ? slots_host[b] : b;
    if (m->host_pos[sl] < 1) p += "slot " + std::to_string(sl) + " holds no prompt; ";
  }
  if (!p.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, p);
  if (noalloc && !m->noalloc_scratch) return fail(QD_ERR_DEVICE, "the fixed sampler scratch has no device address");
  hipStream_t st = (hipStream_t)stream;
  const Plan& P = m->P;
  char* na = static_cast<char*>(m->noalloc_scratch);
  QDCHK(stage_wait(m));
  unsigned long long* hs = stage_seeds(m);
  std::memcpy(hs, seeds_host, (size_t)B * 8);
  unsigned long long* ds = noalloc ? reinterpret_cast<unsigned long long*>(na + NA_SEEDS)
                                   : m->ws<unsigned long long>(P.seeds);
  HIPCHK(hipMemcpyAsync(ds, hs, (size_t)B * 8, hipMemcpyHostToDevice, st));
  const int* row_slot = nullptr;
  if (slots_host) {
    int* hsl = stage_slots(m);
    std::memcpy(hsl, slots_host, (size_t)B * 4);
    int* dsl = noalloc ? reinterpret_cast<int*>(na + NA_SLOTS) : m->ws<int>(P.slot_map);
    HIPCHK(hipMemcpyAsync(dsl, hsl, (size_t)B * 4, hipMemcpyHostToDevice, st));
    row_slot = dsl;
  }
  QDCHK(stage_mark(m, st));
  SampleArgs a{};
  a.logits = logits_dev; a.ldl = m->d.V;
  a.counts = m->ws<int>(P.tok_counts);
  a.row_slot = row_slot;
  a.draws = m->ws<int>(P.draws);
  a.seeds = ds;
  a.next_ids = next_ids_dev;
  a.V = m->d.V; a.top_k = q.top_k;
  a.temperature = q.temperature; a.min_p = q.min_p; a.top_p = q.top_p;
  a.repeat_penalty = q.repeat_penalty; a.presence_penalty = q.presence_penalty;
  a.frequency_penalty = q.frequency_penalty;
  if (noalloc) {
    // the array keeps the last call's contents: the histograms and counters the kernels
    // accumulate into are cleared by a fill kernel (no memset node, so capture is safe)
    a.z = reinterpret_cast<float*>(na + NA_Z);
    a.cand = reinterpret_cast<unsigned long long*>(na + NA_CAND);
    a.hist = reinterpret_cast<unsigned int*>(na + NA_HIST);
    a.rowmax = reinterpret_cast<unsigned int*>(na + NA_ROWMAX);
    a.ncand = reinterpret_cast<int*>(na + NA_NCAND);
    HIPCHK(launch_fill_i32(reinterpret_cast<int*>(na + NA_HIST),
                           (int)((NA_SEEDS - NA_HIST) / 4), 0, st));
  } else {
    a.z = m->ws<float>(P.samp_z);
    a.rowmax = m->ws<unsigned int>(P.smp_rowmax);
    a.hist = m->ws<unsigned int>(P.smp_hist);
    a.ncand = m->ws<int>(P.smp_ncand);
    a.cand = m->ws<unsigned long long>(P.smp_cand);
  }
  HIPCHK(launch_sample(a, B, st));
  return QD_OK;
}
}  // namespace

qd_status qd_sample(qd_model* m, int32_t B, const int32_t* slots_host, const qd_sampling* params,
                    const uint64_t* seeds_host, const float* logits_dev, int32_t* next_ids_dev,
                    qd_stream stream) {
  return sample_impl(m, B, slots_host, params, seeds_host, logits_dev, next_ids_dev, stream, false);
}

qd_status qd_sample_noalloc(qd_model* m, int32_t B, const int32_t* slots_host,
                            const qd_sampling* params, const uint64_t* seeds_host,
                            const float* logits_dev, int32_t* next_ids_dev, qd_stream stream) {
  return sample_impl(m, B, slots_host, params, seeds_host, logits_dev, next_ids_dev, stream, true);
}

qd_status qd_generate_greedy(qd_model* m, int32_t B, const int32_t* prompt_ids_host,
                             const int32_t* lens_host, int32_t max_new_tokens, int32_t eos_id,
                             int32_t* out_ids_host, int32_t* n_out_host, qd_stats* stats,
                             qd_stream stream) {
  g_err.clear();
  if (!m) return fail(QD_ERR_INVALID_ARGUMENTS, "model is NULL");
  std::string p;
  if (B < 1 || B > m->lim.max_batch) p += "B must be in [1, max_batch]; ";
  if (max_new_tokens < 1) p += "max_new_tokens must be >= 1; ";
  if (!prompt_ids_host || !lens_host || !out_ids_host || !n_out_host) p += "NULL pointer argument; ";
  if (!p.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, p);
  std::vector<int> lens(lens_host, lens_host + B);
  long total = 0;
  int need = 0;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < 1) return fail(QD_ERR_INVALID_ARGUMENTS, "empty prompt for sequence " + std::to_string(b));
    total += lens[b];
    need = std::max(need, lens[b] + max_new_tokens - 1);
  }
  if (need > QD_MAX_CONTEXT)
    return fail(QD_ERR_CONTEXT_CEILING, "prompt + max_new_tokens needs " + std::to_string(need) +
                                            " positions, above the ceiling " + std::to_string(QD_MAX_CONTEXT));
  if (need > m->lim.max_ctx || max_new_tokens > m->lim.max_ctx)
    return fail(QD_ERR_INVALID_ARGUMENTS, "prompt + max_new_tokens needs " + std::to_string(need) +
                                              " positions, model loaded with max_ctx " + std::to_string(m->lim.max_ctx));
  if (total > m->lim.max_prefill_tokens)
    return fail(QD_ERR_INVALID_ARGUMENTS, "prompt tokens exceed max_prefill_tokens");
  const std::string e = check_ids(prompt_ids_host, total, m->d.V);
  if (!e.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, e);

  hipStream_t st = (hipStream_t)stream;
  const Plan& P = m->P;
  int* ids_dev = m->ws<int>(P.ids);
  int* next_ids = m->ws<int>(P.next_ids);
  {
    qd_status sw = stage_wait(m);
    if (sw != QD_OK) return sw;
    std::memcpy(m->hstage, prompt_ids_host, (size_t)total * 4);
    HIPCHK(hipMemcpyAsync(ids_dev, m->hstage, total * 4, hipMemcpyHostToDevice, st));
  }
  HIPCHK(launch_fill_i32(m->ws<int>(P.step), 1, 0, st));
  HIPCHK(hipEventRecord(m->ev[0], st));
  qd_status s = enqueue_prefill(m, B, ids_dev, lens, nullptr, next_ids, true, st);
  if (s != QD_OK) return s;
  HIPCHK(hipEventRecord(m->ev[1], st));
  const int steps = max_new_tokens - 1;
  if (steps > 0) {
    int nsplit, split_len;
    // round the context up so one captured graph serves many calls
    const int ctx_cap = std::min(m->lim.max_ctx, ((need + 255) / 256) * 256);
    attn_split(ctx_cap, P.nsplit_cap, m->attn_max_splits, m->attn_min_chunks, attn_occupancy_for(m, B, ctx_cap), B * m->d.KV, &nsplit, &split_len);
    const int waves = attn_waves_for(m, B, ctx_cap);
    // decode steps replayed from captured graphs of GEN_GRAPH_STEPS consecutive steps (the
    // positions and the step counter live on the device), the remainder one step each
    auto graph_for = [&](int n, hipGraphExec_t* out) -> qd_status {
      auto key = std::make_tuple(B, nsplit, split_len * 16 + waves, n);
      auto it = m->graphs.find(key);
      if (it != m->graphs.end()) {
        *out = it->second;
        return QD_OK;
      }
      hipGraph_t graph;
      HIPCHK(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
      qd_status cs = QD_OK;
      for (int i = 0; i < n && cs == QD_OK; ++i)
        cs = enqueue_decode(m, B, next_ids, nullptr, next_ids, true, nsplit, split_len, waves, m->cap_stream);
      hipError_t ee = hipStreamEndCapture(m->cap_stream, &graph);
      if (cs != QD_OK) return cs;
      if (ee != hipSuccess) return fail(QD_ERR_DEVICE, std::string("hipStreamEndCapture: ") + hipGetErrorString(ee));
      hipGraphExec_t exec = nullptr;
      HIPCHK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
      HIPCHK(hipGraphDestroy(graph));
      m->graphs[key] = exec;
      *out = exec;
      return QD_OK;
    };
    const int multi = steps / GEN_GRAPH_STEPS, rest = steps % GEN_GRAPH_STEPS;
    hipGraphExec_t gm = nullptr, g1 = nullptr;
    if (multi) QDCHK(graph_for(GEN_GRAPH_STEPS, &gm));
    if (rest) QDCHK(graph_for(1, &g1));
    for (int i = 0; i < multi; ++i) HIPCHK(hipGraphLaunch(gm, st));
    for (int i = 0; i < rest; ++i) HIPCHK(hipGraphLaunch(g1, st));
  }
  HIPCHK(hipEventRecord(m->ev[2], st));
  HIPCHK(hipMemcpy2DAsync(out_ids_host, (size_t)max_new_tokens * 4, m->ws<int>(P.out_ids),
                          (size_t)m->lim.max_ctx * 4, (size_t)max_new_tokens * 4, B,
                          hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  for (int b = 0; b < B; ++b) {
    m->host_pos[b] = lens[b] + max_new_tokens - 1;
    int n = max_new_tokens;
    if (eos_id >= 0)
      for (int k = 0; k < max_new_tokens; ++k)
        if (out_ids_host[(size_t)b * max_new_tokens + k] == eos_id) {
          n = k + 1;
          break;
        }
    n_out_host[b] = n;
  }
  if (stats) {
    float t0 = 0, t1 = 0;
    HIPCHK(hipEventElapsedTime(&t0, m->ev[0], m->ev[1]));
    HIPCHK(hipEventElapsedTime(&t1, m->ev[1], m->ev[2]));
    stats->prefill_us = t0 * 1e3;
    stats->decode_us = t1 * 1e3;
    stats->steps = steps;
    stats->n_prompt_tokens = (int)total;
  }
  return QD_OK;
}

qd_status qd_profile_kernels(qd_model* m, int32_t B, int32_t iters, float* us_out,
                             qd_stream stream) {
  g_err.clear();
  if (!m || !us_out) return fail(QD_ERR_INVALID_ARGUMENTS, "NULL argument");
  if (B < 1 || B > m->lim.max_batch) return fail(QD_ERR_INVALID_ARGUMENTS, "B must be in [1, max_batch]");
  if (iters < 1) return fail(QD_ERR_INVALID_ARGUMENTS, "iters must be >= 1");
  int ctx = 0;
  for (int b = 0; b < B; ++b) {
    if (m->host_pos[b] >= m->lim.max_ctx)
      return fail(QD_ERR_INVALID_ARGUMENTS, "slot " + std::to_string(b) + " is full (max_ctx)");
    ctx = std::max(ctx, m->host_pos[b] + 1);
  }
  int nsplit, split_len;
  attn_split(ctx, m->P.nsplit_cap, m->attn_max_splits, m->attn_min_chunks, attn_occupancy_for(m, B, ctx), B * m->d.KV, &nsplit, &split_len);
  const int waves = attn_waves_for(m, B, ctx);
  hipStream_t st = (hipStream_t)stream;
  int* scratch_ids = m->ws<int>(m->P.ids);   // prompt-id area doubles as the profiling id list
  HIPCHK(launch_fill_i32(scratch_ids, B, 0, st));
  int* scratch_next = m->ws<int>(m->P.last_rows);  // [max_batch], used by prefill only
  for (int k = 0; k < QD_PROF_COUNT; ++k) {
    // one warm launch, then the timed ones
    for (int rep = 0; rep < 2; ++rep) {
      const int n = rep == 0 ? 1 : iters;
      if (rep == 1) HIPCHK(hipEventRecord(m->ev[0], st));
      for (int i = 0; i < n; ++i) {
        switch (k) {
          case QD_PROF_EMBED:
            HIPCHK(launch_embed(scratch_ids, B, m->w<int8_t>(m->P.emb_q), m->w<float>(m->P.emb_s),
                                m->d.d, m->d.V, m->ws<bf16_t>(m->P.x), st));
            break;
          case QD_PROF_QKV: QDCHK(dec_qkv(m, i % m->d.L, B, st)); break;
          case QD_PROF_ATTN: QDCHK(dec_attn(m, i % m->d.L, B, nsplit, split_len, waves, st)); break;
          case QD_PROF_O: QDCHK(dec_o(m, i % m->d.L, B, st, nsplit)); break;
          case QD_PROF_GATEUP: QDCHK(dec_gateup(m, i % m->d.L, B, st)); break;
          case QD_PROF_DOWN: QDCHK(dec_down(m, i % m->d.L, B, st)); break;
          default:
            QDCHK(enqueue_lm_head(m, m->ws<bf16_t>(m->P.x), nullptr, B, B, nullptr, scratch_next,
                                  false, false, st));
        }
      }
      if (rep == 1) HIPCHK(hipEventRecord(m->ev[1], st));
    }
    HIPCHK(hipEventSynchronize(m->ev[1]));
    float ms = 0;
    HIPCHK(hipEventElapsedTime(&ms, m->ev[0], m->ev[1]));
    us_out[k] = ms * 1e3f / iters;
  }
  return QD_OK;
}

qd_status qd_run_op(qd_model* m, int32_t op, int32_t layer, int32_t B, const void* in_dev,
                    const void* resid_dev, void* out_dev, int32_t* ids_out_dev, qd_stream stream) {
  g_err.clear();
  if (!m) return fail(QD_ERR_INVALID_ARGUMENTS, "model is NULL");
  std::string p;
  if (op < 0 || op >= QD_OP_COUNT) p += "unknown op " + std::to_string(op) + "; ";
  if (layer < 0 || layer >= m->d.L) p += "layer out of range; ";
  if (B < 1 || B > m->lim.max_batch) p += "B must be in [1, max_batch]; ";
  if (!in_dev || !out_dev) p += "in_dev and out_dev must be set; ";
  if ((op == QD_OP_O || op == QD_OP_DOWN) && !resid_dev) p += "resid_dev must be set for this op; ";
  if (op == QD_OP_LMHEAD && !ids_out_dev) p += "ids_out_dev must be set for the LM head; ";
  if (!p.empty()) return fail(QD_ERR_INVALID_ARGUMENTS, p);
  const Dims& d = m->d;
  const Plan& P = m->P;
  hipStream_t st = (hipStream_t)stream;
  auto put = [&](size_t off, const void* src, size_t bytes) -> hipError_t {
    return hipMemcpyAsync(m->WS + off, src, bytes, hipMemcpyDeviceToDevice, st);
  };
  auto get = [&](size_t off, size_t bytes) -> hipError_t {
    return hipMemcpyAsync(out_dev, m->WS + off, bytes, hipMemcpyDeviceToDevice, st);
  };
  const size_t xb = (size_t)B * d.d * 2;
  switch (op) {
    case QD_OP_EMBED:
      // the decode step's embedding launch, without the sampler's occurrence counts
      HIPCHK(launch_embed(static_cast<const int*>(in_dev), B, m->w<int8_t>(P.emb_q),
                          m->w<float>(P.emb_s), d.d, d.V, static_cast<bf16_t*>(out_dev), st));
      break;
    case QD_OP_QKV:
      HIPCHK(put(P.x, in_dev, xb));
      QDCHK(dec_qkv(m, layer, B, st));
      HIPCHK(get(P.qkv, (size_t)B * d.NQKV * 2));
      break;
    case QD_OP_O:
      HIPCHK(put(P.attn, in_dev, (size_t)B * d.HD * 2));
      HIPCHK(put(P.x, resid_dev, xb));
      QDCHK(dec_o(m, layer, B, st));
      HIPCHK(get(P.x, xb));
      break;
    case QD_OP_GATEUP:
      HIPCHK(put(P.x, in_dev, xb));
      QDCHK(dec_gateup(m, layer, B, st));
      HIPCHK(get(P.act, (size_t)B * d.I * 2));
      break;
    case QD_OP_DOWN:
      HIPCHK(put(P.act, in_dev, (size_t)B * d.I * 2));
      HIPCHK(put(P.x, resid_dev, xb));
      QDCHK(dec_down(m, layer, B, st));
      HIPCHK(get(P.x, xb));
      break;
    default:
      HIPCHK(put(P.x, in_dev, xb));
      QDCHK(enqueue_lm_head(m, m->ws<bf16_t>(P.x), nullptr, B, B, static_cast<float*>(out_dev),
                            ids_out_dev, false, false, st));
      break;
  }
  return QD_OK;
}

qd_status qd_set_tuning(qd_model* m, int32_t knob, int32_t value) {
  g_err.clear();
  if (!m) return fail(QD_ERR_INVALID_ARGUMENTS, "model is NULL");
  if (value < 0 || (value < 1 && knob != QD_TUNE_ATTN_MERGE_LAST && knob != QD_TUNE_ATTN_WAVES &&
                    knob != QD_TUNE_GEMM_SPLITS &&
                    knob != QD_TUNE_ATTN_OCCUPANCY && knob != QD_TUNE_SKINNY_NORM &&
                    knob != QD_TUNE_PREFILL_GEMM && knob != QD_TUNE_SKINNY_XSTAGE &&
                    knob != QD_TUNE_FLASH_ROWS))
    return fail(QD_ERR_INVALID_ARGUMENTS, "value out of range");
  switch (knob) {
    case QD_TUNE_ATTN_MAX_SPLITS: m->attn_max_splits = value; break;
    case QD_TUNE_ATTN_MIN_CHUNKS: m->attn_min_chunks = value; break;
    case QD_TUNE_ATTN_MERGE_LAST:
      if (value > 2) return fail(QD_ERR_INVALID_ARGUMENTS, "merge mode must be 0, 1 or 2");
      m->attn_merge_last = value;
      break;
    case QD_TUNE_SKINNY_NORM:
      if (value > 1) return fail(QD_ERR_INVALID_ARGUMENTS, "skinny norm mode must be 0 or 1");
      m->skinny_norm = value;
      break;
    case QD_TUNE_FLASH_ROWS:
      if (value != 0 && value != 64 && value != 128)
        return fail(QD_ERR_INVALID_ARGUMENTS, "prefill attention tile rows must be 0, 64 or 128");
      m->flash_rows = value;
      break;
    case QD_TUNE_SKINNY_XSTAGE:
      if (value > 1) return fail(QD_ERR_INVALID_ARGUMENTS, "activation staging mode must be 0 or 1");
      m->skinny_xstage = value;
      break;
    case QD_TUNE_PREFILL_GEMM:
      if (value > 1) return fail(QD_ERR_INVALID_ARGUMENTS, "prefill GEMM mode must be 0 or 1");
      m->gemm_ks = value;
      m->gemm_rope = value;
      break;
    case QD_TUNE_ATTN_OCCUPANCY:
      if (value > 8) return fail(QD_ERR_INVALID_ARGUMENTS, "attention occupancy must be 0..8");
      m->attn_occupancy = value;
      break;
    case QD_TUNE_GEMM_SPLITS:
      if (value > 8) return fail(QD_ERR_INVALID_ARGUMENTS, "at most 8 GEMM splits");
      m->gemm_splits = value;
      break;
    case QD_TUNE_SKINNY_SPLIT:
      if (value > 3) return fail(QD_ERR_INVALID_ARGUMENTS, "skinny split mode must be 1, 2 or 3");
      m->skinny_split = value;
      break;
    case QD_TUNE_ATTN_WAVES:
      if (value != 0 && value != 4 && value != 8)
        return fail(QD_ERR_INVALID_ARGUMENTS, "attention waves must be 0 (by batch), 4 or 8");
      m->attn_waves = value;
      break;
    default: return fail(QD_ERR_INVALID_ARGUMENTS, "unknown knob");
  }
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  m->graphs.clear();
  return QD_OK;
}

void qd_free(qd_model* m) {
  if (!m) return;
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  for (int i = 0; i < 3; ++i)
    if (m->ev[i]) (void)hipEventDestroy(m->ev[i]);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  if (m->stage_ev) {
    (void)hipEventSynchronize(m->stage_ev);
    (void)hipEventDestroy(m->stage_ev);
  }
  if (m->hstage) (void)hipHostFree(m->hstage);
  delete m;
}

}  // extern "C"
