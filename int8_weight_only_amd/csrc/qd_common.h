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

enum Epilogue { EPI_STORE = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_LOGITS = 3 };

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
  int* pos;                          // optional [nb]: incremented by the last block
  int* out_ids; int out_ld;          // optional: out_ids[b*out_ld + *step] = id
  unsigned long long* part_keys;     // [nb][LM_MAX_GRID] per-work-group best keys
  int* step;                         // device step counter (read when out_ids is set)
  int bump_step;                     // the last block increments *step
  int batch0;                        // batch index of row 0 of this launch (for pos/out_ids)
};

struct GemmArgs {
  const bf16_t* A; int lda;   // [M][K] bf16 activations
  const int8_t* W;            // [N][K]
  const float* scale;         // [N]
  int M, N, K;
  int epi;                    // EPI_STORE / EPI_RESID / EPI_SILU
  bf16_t* out; int ldo;
  float* part;                // split-K partial sums [splits][M][N] (fp32), PART_FLOATS max
  int splits;                 // set by the launcher
};
constexpr size_t GEMM_PART_FLOATS = (size_t)8 << 20;  // 32 MiB of split-K partials

struct RopeArgs {
  bf16_t* qkv; int ldqkv;     // [M][(H+2KV)*D]; q heads rewritten in place
  const float* q_gain; const float* k_gain; float eps;
  const float2* rope;         // [max_ctx][D/2] (cos, sin)
  const int* row_slot; const int* row_pos;  // per row
  bf16_t* kcache; bf16_t* vcache;           // this layer's [slots][KV][ctx][D]
  int H, KV, D, max_ctx, M;
};


// decode attention with QK-norm, RoPE and the KV write fused in; splits of the context
// are merged by the last split to finish (per-(row, KV head) counters)
struct AttnDecArgs {
  const bf16_t* qkv; int ldqkv;   // raw q|k|v projections, row b at qkv + b*ldqkv
  const float* q_gain; const float* k_gain; float eps;
  const float2* rope;             // [max_ctx][D/2]
  const int* pos;                 // [B] position of the token being decoded (slot b = row b)
  bf16_t* kcache; bf16_t* vcache; // this layer's [slots][KV][ctx][D]
  int H, KV, D, max_ctx, B;
  int split_len, nsplit;
  int nwaves;                     // 4, 8 or 16 waves per work-group (8, 16 only when G*D <= 512)
  int merge_last;                 // 1: the last split merges (fence + counter); 0: merge kernel
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
  const int4* tiles;                           // [grid.x]
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
                        bf16_t* x, hipStream_t st);
hipError_t launch_rmsnorm(const bf16_t* x, int M, int d, const float* g, float eps, bf16_t* y,
                          hipStream_t st);
hipError_t launch_gemv(const GemvArgs& a, int epi, hipStream_t st);
hipError_t launch_skinny(const GemvArgs& a, int epi, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_qk_rope(const RopeArgs& a, hipStream_t st);
hipError_t launch_attention_decode(const AttnDecArgs& a, hipStream_t st);
hipError_t launch_flash_prefill(const FlashArgs& a, int n_tiles, hipStream_t st);
hipError_t launch_set_positions(int* pos, const int* lens, int n, hipStream_t st);
hipError_t launch_iota(int* p, int n, hipStream_t st);

}  // namespace qd
