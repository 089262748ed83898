// Shared device helpers and the launcher interface between the host API
// (qd_api.hip) and the kernels (qd_kernels.hip).  Internal: not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

typedef uint16_t bf16_t;  // bf16 bit pattern

// fused gate/up matrices store rows in blocks of GU_BLOCK gate rows followed by the
// GU_BLOCK matching up rows, so one tile holds both halves of SiLU(gate) * up
constexpr int GU_BLOCK = 16;
// decode attention: positions per work-group chunk
constexpr int ATT_CHUNK = 64;
constexpr int ATT_MAX_SPLITS = 256;

__host__ __device__ inline int gu_row(int j, int half) {  // logical row j of gate(0)/up(1)
  return (j / GU_BLOCK) * (2 * GU_BLOCK) + half * GU_BLOCK + (j % GU_BLOCK);
}

// ---- launch parameter blocks ------------------------------------------------------------

enum Epilogue { EPI_STORE = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_LOGITS = 3,
                // prefill GEMM only: each split-K work-group stores its fp32 partial in
                // [split][M][N]; k_resid_norm adds them into the residual (scaled) and
                // normalizes the result for the next projection
                EPI_PART = 4 };

struct GemvArgs {
  const bf16_t* x;      // [nb][ldx] input activations (pre-norm when gain != null)
  int ldx;
  const int* x_rows;    // optional: batch b reads row x_rows[b] of x
  const float* gain;    // RMSNorm gain of the prologue, or null (x already normalized)
  float eps;
  const int8_t* W;      // [N][K] int8 codes (rows possibly gate/up interleaved)
  const float* scale;   // [N]
  int N, K;
  int nb;               // batch rows in this launch (GEMV 1, skinny MFMA 1..64)
  bf16_t* out; int ldo; // EPI_STORE/EPI_SILU: output; EPI_RESID: residual updated in place
  // EPI_LOGITS
  float* logits; int ldl;            // optional fp32 logits [nb][ldl]
  unsigned int* done;                // completion counter, zero on entry
  int* next_ids;                     // [nb] greedy ids out
  int* pos;                          // optional [slots]: the row's slot position is incremented
  const int* row_slot;               // optional [nb]: KV slot of row b for pos (NULL: slot b)
  int* out_ids; int out_ld;          // optional: out_ids[b*out_ld + *step] = id
  unsigned long long* part_keys;     // [nb][LM_MAX_GRID] per-work-group best keys
  int* step;                         // device step counter (read when out_ids is set)
  int bump_step;                     // the last block increments *step
  int batch0;                        // batch index of row 0 of this launch (for pos/out_ids)
  // skinny split-K (EPI_STORE / EPI_RESID / EPI_SILU): ksplit work-groups per channel tile
  int ksplit;                        // <= 1: one work-group per tile
  float* kpart;                      // [tiles][ksplit][CTW][16*TT tokens x 16 channels] partials
  unsigned int* kcnt;                // [tiles] arrival counters, zero on entry, reset by the last
  int no_xstage;                     // skinny, up to 16 rows: 1 = activations loaded straight in
                                     // the MFMA operand layout instead of row-contiguous + LDS
  // B=1 EPI_RESID with att_ns > 0 (the O projection after a decode attention that left its
  // att_ns split partials): the activation row is merged from part_o [K/att_D][att_ns][att_D]
  // and part_ml [K/att_D][att_ns][2] (base-2 maxima and sums) instead of read from x
  const float* att_po; const float* att_ml; int att_ns; int att_D;
};
constexpr int ATT_DEFER_MAX_SPLITS = 8;  // most splits whose merge the O projection takes
constexpr int SKINNY_MAX_SPLIT = 16;
constexpr int SKINNY_MAX_TILES = 4096;

struct RopeArgs {
  bf16_t* qkv; int ldqkv;     // [M][(H+2KV)*D]; q heads rewritten in place
  const float* q_gain; const float* k_gain; float eps;
  const float2* rope;         // [max_ctx][D/2] (cos, sin)
  const int* row_slot; const int* row_pos;  // per row
  bf16_t* kcache; bf16_t* vcache;           // this layer's [slots][KV][ctx][D]
  int H, KV, D, max_ctx, M;
};

struct GemmArgs {
  const bf16_t* A; int lda;   // [M][K] bf16 activations
  const int8_t* W;            // [N][K]
  const float* scale;         // [N]
  int M, N, K;
  int epi;                    // EPI_STORE / EPI_RESID / EPI_SILU
  bf16_t* out; int ldo;
  float* part;                // split-K tile partials [tiles][splits][64 x 64] (fp32)
  unsigned int* cnt;          // split-K arrival counters per tile, zero on entry
  int splits;                 // in: most split-K ways (0: launcher's default); set by the launcher
  int defer;                  // EPI_RESID with split-K: store partials (EPI_PART) instead of
                              // merging them in-kernel; the caller runs k_resid_norm next
  int use_big = 1;            // 0: never the 128x128-tile kernel (tuning)
  int use_ks = 1;             // 0: never the k-sliced few-row kernel (tuning)
  // EPI_STORE of the q|k|v projection: the 32x128-, 128x128- and 256x256-tile kernels may run
  // the QK-norm, RoPE and K/V cache writes of the heads in a tile in their epilogues (rope.qkv is not read: the
  // projection's rows are the tile; q heads go to out, K and V heads only to the caches)
  int fuse_rope = 0;
  RopeArgs rope{};
};
constexpr size_t GEMM_PART_FLOATS = (size_t)8 << 20;  // 32 MiB of split-K partials



// decode attention with QK-norm, RoPE and the KV write fused in; splits of the context
// are merged by the last split to finish (per-(row, KV head) counters)
struct AttnDecArgs {
  const bf16_t* qkv; int ldqkv;   // raw q|k|v projections, row b at qkv + b*ldqkv
  const float* q_gain; const float* k_gain; float eps;
  const float2* rope;             // [max_ctx][D/2]
  const int* pos;                 // [slots] position of the token being decoded, per KV slot
  const int* row_slot;            // [B] KV slot of row b (NULL: slot b)
  bf16_t* kcache; bf16_t* vcache; // this layer's [slots][KV][ctx][D]
  int H, KV, D, max_ctx, B;
  int split_len, nsplit;
  int nwaves;                     // 4 or 8 waves per work-group (8 only when G*D <= 512)
  int merge_last;                 // 1: the last split merges (agent-coherent partials + counter); 0: merge
                                  // kernel; 2: the partials are left for the next kernel to merge
  float* part_o;                  // [B][H][nsplit][D]
  float* part_ml;                 // [B][H][nsplit][2]
  unsigned int* counters;         // [B][KV], zero on entry; the merging split resets it
  bf16_t* out; int ldo;           // [B][H*D]
};

// prefill attention: a work-group owns a tile of up to 64 query rows of one sequence and
// one query head; tiles are described by (first row, slot, first position, rows)
struct FlashArgs {
  const bf16_t* q; int ldq;                    // roped q rows; head h at q + r*ldq + h*D
  const bf16_t* kcache; const bf16_t* vcache;  // this layer's [slots][KV][ctx][D]
  const int4* tiles;                           // [grid.y]: (row0, slot, pos0, rows)
  int H, KV, D, max_ctx;
  bf16_t* out; int ldo;                        // [M][H*D]
};
constexpr int FLASH_ROWS = 64;

constexpr int LM_MAX_GRID = 1024;  // work-groups of the LM-head GEMV (row blocks looped)

// ---- launchers (qd_kernels.hip) ------------------------------------------------------------
hipError_t launch_quantize_rows(const float* w, int rows, int cols, int8_t* q, float* s,
                                int dst_row0, int gu_half, hipStream_t st);
hipError_t launch_rope_table(float2* tab, int max_ctx, int D, float theta, hipStream_t st);
hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st);
hipError_t launch_embed(const int* ids, int M, const int8_t* E, const float* Es, int d, int V,
                        bf16_t* x, hipStream_t st, int* counts = nullptr,
                        const int* row_slot = nullptr);
hipError_t launch_rmsnorm(const bf16_t* x, int M, int d, const float* g, float eps, bf16_t* y,
                          hipStream_t st);
hipError_t launch_gemv(const GemvArgs& a, int epi, hipStream_t st);
hipError_t launch_skinny(const GemvArgs& a, int epi, hipStream_t st);
// whether launch_skinny can fold the RMSNorm (gain set) for nb rows of a K-long input
bool skinny_norm_ok(int nb, int K, int epi, int ksplit);
// *splits_used (nullable) receives the split-K ways; with a.defer and more than one
// split, the residual is not yet updated: launch_resid_norm with that count must follow
// rope_done (optional): set to 1 when the launch also did the QK-norm / RoPE / cache writes
// that a.fuse_rope asked for, else 0 (the caller then runs launch_qk_rope)
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st, int* splits_used = nullptr,
                       int* rope_done = nullptr);
// x[m] = bf16(x[m] + bf16(scale * sum_s part[s][m])) in split order, then
// y[m] = RMSNorm(x[m]) * g; splits in {2, 4, 8}
hipError_t launch_resid_norm(bf16_t* x, int M, int d, const float* part, int splits,
                             const float* scale, const float* g, float eps, bf16_t* y,
                             hipStream_t st);
hipError_t launch_qk_rope(const RopeArgs& a, hipStream_t st);

// ---- sampled decode: one work-group per logits row ----------------------------------------
constexpr int SMP_MAXK = 1024;  // largest top_k the device sampler takes
struct SampleArgs {
  const float* logits; int ldl;     // [B][ldl] fp32 logits
  float* z;                         // scratch [B][V]: penalized, tempered logits
  const int* counts;                // [slots][V] occurrences of each token in the sequence
  const int* row_slot;              // [B] KV slot of row b (NULL: slot b)
  int* draws;                       // [slots] draws so far (the Philox counter)
  const unsigned long long* seeds;  // [B] Philox key of each row's sequence
  int* next_ids;                    // [B] drawn ids out
  int V, top_k;
  float temperature, min_p, top_p, repeat_penalty, presence_penalty, frequency_penalty;
  // per-row state of one call, zero on entry and cleared again by the call's last kernel
  unsigned int* rowmax;             // [B] largest key of the row
  unsigned int* hist;               // [B][256] distance histogram
  int* ncand;                       // [B] gathered candidates
  unsigned long long* cand;         // [B][SMP_CAND_G] gathered (key, ~id)
};
constexpr int SMP_CAND_G = 8192;
hipError_t launch_sample(const SampleArgs& a, int B, hipStream_t st);
// Fixed scratch of the sampler for callers that cannot allocate (qd_sample_noalloc): a
// file-scope device array in qd_sample.hip, one per device.  Capacity: NOALLOC_MAX_ROWS rows
// and rows x vocab <= NOALLOC_Z_FLOATS.  Layout (byte offsets, each 256-aligned):
constexpr int NOALLOC_MAX_ROWS = 16;
constexpr size_t NOALLOC_Z_FLOATS = size_t(1) << 21;
constexpr size_t NA_Z = 0;                                                  // fp32 [rows][V]
constexpr size_t NA_CAND = NA_Z + NOALLOC_Z_FLOATS * 4;                     // u64 [16][8192]
constexpr size_t NA_HIST = NA_CAND + size_t(NOALLOC_MAX_ROWS) * SMP_CAND_G * 8;  // u32 [16][256]
constexpr size_t NA_ROWMAX = NA_HIST + size_t(NOALLOC_MAX_ROWS) * 256 * 4;  // u32 [16]
constexpr size_t NA_NCAND = NA_ROWMAX + 256;                                // i32 [16]
constexpr size_t NA_SEEDS = NA_NCAND + 256;                                 // u64 [16]
constexpr size_t NA_SLOTS = NA_SEEDS + 256;                                 // i32 [16]
constexpr size_t NOALLOC_SCRATCH_BYTES = NA_SLOTS + 256;
// The current device's address of that array (looked up with hipGetSymbolAddress on the
// first call per device, then cached); the device must be current.
hipError_t sample_scratch_address(void** out);
// zeroes counts[slot][:] and draws[slot] for slots[0..n) (NULL: slots 0..n-1)
hipError_t launch_reset_seq(int* counts, int* draws, const int* slots, int n, int V, hipStream_t st);
hipError_t launch_attention_decode(const AttnDecArgs& a, hipStream_t st);
// work-groups of the decode attention kernel for (D, G, waves) resident on one CU
hipError_t attention_decode_residency(int D, int G, int nwaves, int* blocks_per_cu);
// tile_rows: FLASH_ROWS or 2 * FLASH_ROWS (head dim up to 128), as the tiles were cut
hipError_t launch_flash_prefill(const FlashArgs& a, int n_tiles, int tile_rows, hipStream_t st);
hipError_t launch_set_positions(int* pos, const int* lens, const int* slots, int n, hipStream_t st);
hipError_t launch_iota(int* p, int n, hipStream_t st);


}  // namespace qd
