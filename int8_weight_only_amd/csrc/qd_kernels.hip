// HIP kernels for the int8 weight-only Qwen3-family decoder step, written for
// gfx950 (CDNA4, wave64).  The decoder follows "Model-agnostic LLM inference",
// section "Supported models"; the int8 weights with one scale per row follow the
// section "The quantized load cache" of the same page.
//
// Rounding: every tensor the model produces is rounded to bf16 (round to nearest
// even) at the same points as the CPU oracle: embedding rows, RMSNorm outputs,
// projection outputs, QK-norm and RoPE outputs, attention outputs, residual sums,
// SiLU(gate)*up.  Logits stay fp32.  Accumulation is fp32.
#include "qd_device.h"

namespace qd {

// ------------------------------------------------------------------------------------------
// load time: per-row symmetric int8 quantization (bit-exact contract)
//   s = absmax / 127 (IEEE fp32 division), q = clamp(rint(w / s), -127, 127); zero row -> 0
__global__ __launch_bounds__(256) void k_quantize_rows(const float* __restrict__ w, int cols,
                                                       int8_t* __restrict__ q,
                                                       float* __restrict__ s, int dst_row0,
                                                       int gu_half) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const float* wr = w + (size_t)r * cols;
  float amax = 0.0f;
  for (int c = threadIdx.x; c < cols; c += 256) amax = fmaxf(amax, fabsf(wr[c]));
  amax = block_max256(amax, red);
  const float sc = amax / 127.0f;
  const int dr = gu_half >= 0 ? dst_row0 + gu_row(r, gu_half) : dst_row0 + r;
  int8_t* qr = q + (size_t)dr * cols;
  if (threadIdx.x == 0) s[dr] = sc;
  for (int c = threadIdx.x; c < cols; c += 256) {
    int v = 0;
    if (sc != 0.0f) {
      float t = rintf(wr[c] / sc);
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      v = (int)t;
    }
    qr[c] = (int8_t)v;
  }
}

// RoPE table: (cos, sin) of p * theta^(-2i/D) computed in float64, stored fp32
__global__ void k_rope_table(float2* tab, int max_ctx, int D, double theta) {
  const int half = D / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)max_ctx * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)D);
  const double ang = (double)p * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

__global__ void k_fill_i32(int* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void k_iota(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = i;
}
__global__ void k_set_positions(int* pos, const int* lens, const int* slots, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[slots ? slots[i] : i] = lens[i];
}

// ------------------------------------------------------------------------------------------
// embedding gather: x = bf16(code * row scale), product in fp32
// (ids outside [0, V) are clamped into range so a bad id can never read out of bounds;
// the host validates ids wherever it sees them)
// With `counts`, the token is also counted for its sequence (the sampler's penalties):
// counts[slot][t] += 1, slot = row_slot[r] (NULL: r).
__global__ __launch_bounds__(256) void k_embed(const int* __restrict__ ids,
                                               const int8_t* __restrict__ E,
                                               const float* __restrict__ Es, int d, int V,
                                               bf16_t* __restrict__ x, int* counts,
                                               const int* row_slot) {
  const int r = blockIdx.x;
  const int t = min(max(ids[r], 0), V - 1);
  if (counts && threadIdx.x == 0) atomicAdd(counts + (size_t)(row_slot ? row_slot[r] : r) * V + t, 1);
  // the row's scale and every code of it are requested at once (4 codes per thread and pass,
  // passes unrolled, clamped offsets), then converted and stored: one round trip after the
  // id (d is a multiple of 32 and at most 8192)
  constexpr int NP = 8;
  const float s = Es[t];
  const int8_t* er = E + (size_t)t * d;
  uint32_t w[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = 4 * threadIdx.x + 1024 * p;
    w[p] = *reinterpret_cast<const uint32_t*>(er + (c < d ? c : 0));
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = 4 * threadIdx.x + 1024 * p;
    if (c >= d) break;
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v0 = ((int)(w[p] << (24 - 16 * h))) >> 24, v1 = ((int)(w[p] << (16 - 16 * h))) >> 24;
      o[h] = (uint32_t)f2bf((float)v0 * s) | ((uint32_t)f2bf((float)v1 * s) << 16);
    }
    *reinterpret_cast<uint2*>(x + (size_t)r * d + c) = make_uint2(o[0], o[1]);
  }
}

// RMSNorm of M rows, y = bf16(x / sqrt(mean(x^2) + eps) * g) (d % 8 == 0, d <= 8192): one
// row per wave (four per work-group), the row and its gains loaded once into registers
// (CPL 16-byte chunks per lane), a wave reduction, no block barrier.
template <int CPL>
__global__ __launch_bounds__(256) void k_rmsnorm(const bf16_t* __restrict__ x, int M, int d,
                                                 const float* __restrict__ g, float eps,
                                                 bf16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M) return;  // whole waves; no block barrier follows
  const bf16_t* xr = x + (size_t)r * d;
  bf16_t* yr = y + (size_t)r * d;
  const int nch = d >> 3;
  uint4 u[CPL];
  float4 g0[CPL], g1[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {  // clamped (valid) indices: no load in a branch
    const int c = lane + 64 * q;
    const int cc = c < nch ? c : 0;
    u[q] = *reinterpret_cast<const uint4*>(xr + 8 * cc);
    g0[q] = *reinterpret_cast<const float4*>(g + 8 * cc);
    g1[q] = *reinterpret_cast<const float4*>(g + 8 * cc + 4);
  }
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    if (lane + 64 * q < nch) {
      const uint32_t w4[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(w4[j] << 16), hi = __uint_as_float(w4[j] & 0xFFFF0000u);
        ss += lo * lo + hi * hi;
      }
    }
  }
  const float rinv = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + 64 * q;
    if (c < nch) {
      const uint32_t w4[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
      const float gv[8] = {g0[q].x, g0[q].y, g0[q].z, g0[q].w, g1[q].x, g1[q].y, g1[q].z, g1[q].w};
      uint32_t o4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16_t y0 = f2bf(__uint_as_float(w4[j] << 16) * rinv * gv[2 * j]);
        const bf16_t y1 = f2bf(__uint_as_float(w4[j] & 0xFFFF0000u) * rinv * gv[2 * j + 1]);
        o4[j] = (uint32_t)y0 | ((uint32_t)y1 << 16);
      }
      *reinterpret_cast<uint4*>(yr + 8 * c) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
  }
}

// split-K merge of a prefill projection into the residual stream, then the RMSNorm of the
// updated row (one row per wave): x = bf16(x + bf16(scale * (p_0 + p_1 + ... + p_{S-1})))
// with the partials added in split order, y = bf16(x / sqrt(mean(x^2) + eps) * g).  Every
// input of the row (residual, partials, scales, gains) is requested before the first use.
template <int CPL, int S>
__global__ __launch_bounds__(256) void k_resid_norm(bf16_t* __restrict__ x, int M, int d,
                                                    const float* __restrict__ part,
                                                    const float* __restrict__ scale,
                                                    const float* __restrict__ g, float eps,
                                                    bf16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M) return;  // whole waves; no block barrier follows
  bf16_t* xr = x + (size_t)r * d;
  bf16_t* yr = y + (size_t)r * d;
  const int nch = d >> 3;
  uint4 u[CPL];
  float4 p[S][CPL][2], sc[CPL][2];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {  // clamped (valid) indices: no load in a branch
    const int c = lane + 64 * q;
    const int cc = c < nch ? c : 0;
    u[q] = *reinterpret_cast<const uint4*>(xr + 8 * cc);
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
      const float* ps = part + ((size_t)sp * M + r) * d + 8 * cc;
      p[sp][q][0] = *reinterpret_cast<const float4*>(ps);
      p[sp][q][1] = *reinterpret_cast<const float4*>(ps + 4);
    }
    sc[q][0] = *reinterpret_cast<const float4*>(scale + 8 * cc);
    sc[q][1] = *reinterpret_cast<const float4*>(scale + 8 * cc + 4);
  }
  float4 g0[CPL], g1[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + 64 * q;
    const int cc = c < nch ? c : 0;
    g0[q] = *reinterpret_cast<const float4*>(g + 8 * cc);
    g1[q] = *reinterpret_cast<const float4*>(g + 8 * cc + 4);
  }
  float xv[CPL][8];
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const uint32_t w4[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
    const float s8[8] = {sc[q][0].x, sc[q][0].y, sc[q][0].z, sc[q][0].w,
                         sc[q][1].x, sc[q][1].y, sc[q][1].z, sc[q][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.0f;
#pragma unroll
      for (int sp = 0; sp < S; ++sp) {
        const float4& pp = p[sp][q][e >> 2];
        const float pe = (e & 3) == 0 ? pp.x : (e & 3) == 1 ? pp.y : (e & 3) == 2 ? pp.z : pp.w;
        v = sp == 0 ? pe : v + pe;
      }
      const float xo = (e & 1) ? __uint_as_float(w4[e >> 1] & 0xFFFF0000u) : __uint_as_float(w4[e >> 1] << 16);
      xv[q][e] = rbf(xo + rbf(v * s8[e]));
      ss += lane + 64 * q < nch ? xv[q][e] * xv[q][e] : 0.0f;
    }
  }
  const float rinv = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + 64 * q;
    if (c < nch) {
      const float gv[8] = {g0[q].x, g0[q].y, g0[q].z, g0[q].w, g1[q].x, g1[q].y, g1[q].z, g1[q].w};
      uint32_t o4[4], x4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x4[j] = (uint32_t)f2bf(xv[q][2 * j]) | ((uint32_t)f2bf(xv[q][2 * j + 1]) << 16);
        const bf16_t y0 = f2bf(xv[q][2 * j] * rinv * gv[2 * j]);
        const bf16_t y1 = f2bf(xv[q][2 * j + 1] * rinv * gv[2 * j + 1]);
        o4[j] = (uint32_t)y0 | ((uint32_t)y1 << 16);
      }
      *reinterpret_cast<uint4*>(xr + 8 * c) = make_uint4(x4[0], x4[1], x4[2], x4[3]);
      *reinterpret_cast<uint4*>(yr + 8 * c) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
  }
}

// ------------------------------------------------------------------------------------------
// decode GEMV helpers

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long t = shfl_xor_u64(v, o);
    v = t > v ? t : v;
  }
  return v;
}

// LM head tail: each work-group stores its best (value, index) key per batch row; the
// keys are reduced by k_lm_finish in the next launch (the kernel boundary makes them
// visible without a device-wide fence in every work-group).  best is valid in thread b.
__device__ __forceinline__ void lm_head_store(const GemvArgs& a, unsigned long long best, int nb_max) {
  const int tid = threadIdx.x;
  if (tid < a.nb && tid < nb_max) a.part_keys[(size_t)tid * LM_MAX_GRID + blockIdx.x] = best;
}

// one work-group per batch row: reduces that row's keys over the LM-head work-groups and
// writes the greedy id (advancing its position).  The step counter advances once every
// row has read it: in k_lm_finish_step, launched after, or here when there is one row
__global__ __launch_bounds__(256) void k_lm_finish(unsigned long long* keys_, int* next_ids_, int* pos_,
                                                   const int* row_slot_, int* out_ids_, int* step_,
                                                   int nblocks, GemvArgs a) {
  // the pointers come as leading scalar arguments, preloaded into SGPRs at wave launch
  a.part_keys = keys_;
  a.next_ids = next_ids_;
  a.pos = pos_;
  a.row_slot = row_slot_;
  a.out_ids = out_ids_;
  a.step = step_;
  __shared__ unsigned long long red[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  unsigned long long k = 0ull;
  for (int i = tid; i < nblocks; i += 256) {
    const unsigned long long v = a.part_keys[(size_t)b * LM_MAX_GRID + i];
    k = v > k ? v : k;
  }
  k = wave_max_u64(k);
  if (lane == 0) red[wid] = k;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) k = red[w] > k ? red[w] : k;
    k = red[0] > k ? red[0] : k;
    const int id = key_index(k);
    a.next_ids[b] = id;
    if (a.out_ids) a.out_ids[(size_t)(a.batch0 + b) * a.out_ld + *a.step] = id;
    if (a.pos) a.pos[a.row_slot ? a.row_slot[b] : b] += 1;
    // a single row advances the step counter itself (no other work-group reads it)
    if (a.bump_step && gridDim.x == 1) *a.step += 1;
  }
}

__global__ void k_lm_finish_step(int* step) { *step += 1; }

// ------------------------------------------------------------------------------------------
// single-row decode GEMV: y[n] = scale[n] * sum_k x[k] * W[n][k].
// Every wave keeps the whole activation row in registers (lane l owns the 16-element
// chunks l, l+64, ...), so the RMSNorm prologue is a wave reduction with no LDS and no
// block barrier.  The activations and gains are requested first and the first weight
// chunks right after, so the two memory latencies overlap and the norm waits only for its
// own inputs.  A work-group owns 4*R rows (EPI_SILU: R gate rows and their R up rows per
// wave) and loops over row blocks when the grid is capped.
// MERGE (EPI_RESID, the O projection at B = 1): the activation row is the decode
// attention's output, merged here from the attention's split partials (each thread 8 dims,
// all splits requested at once) into LDS, which the waves then read instead of x.  This
// takes the attention kernel's last-split hand-off (store completion, counter, reload)
// off the step's critical path.
// Leading scalar arguments of the prefill GEMMs (k_gemm, k_gemm_ks, k_gemm_dl, k_gemm_big),
// prefill attention (k_flash_prefill) and the prefill QK-norm/RoPE (k_qk_rope): the fields
// their first loads need, preloaded into SGPRs at wave launch.
#define QD_GEMM_PRELOAD_PARAMS                                                                  \
  const bf16_t *A_, const int8_t *W_, const float *scale_, bf16_t *out_, int M_, int N_, int K_, \
      int lda_, int ldo_, int splits_
#define QD_GEMM_PRELOAD_SET(a)                                                                    \
  do {                                                                                            \
    (a).A = A_;                                                                                   \
    (a).W = W_;                                                                                   \
    (a).scale = scale_;                                                                           \
    (a).out = out_;                                                                               \
    (a).M = M_;                                                                                   \
    (a).N = N_;                                                                                   \
    (a).K = K_;                                                                                   \
    (a).lda = lda_;                                                                               \
    (a).ldo = ldo_;                                                                               \
    (a).splits = splits_;                                                                         \
  } while (0)
#define QD_GEMM_PRELOAD_ARGS(a) (a).A, (a).W, (a).scale, (a).out, (a).M, (a).N, (a).K, (a).lda, (a).ldo, (a).splits
#define QD_FLASH_PRELOAD_PARAMS \
  const int4 *tiles_, const bf16_t *q_, const bf16_t *kc_, const bf16_t *vc_, int ldq_, int H_, int KV_, int max_ctx_
#define QD_FLASH_PRELOAD_SET(a) \
  do {                          \
    (a).tiles = tiles_;         \
    (a).q = q_;                 \
    (a).kcache = kc_;           \
    (a).vcache = vc_;           \
    (a).ldq = ldq_;             \
    (a).H = H_;                 \
    (a).KV = KV_;               \
    (a).max_ctx = max_ctx_;     \
  } while (0)
#define QD_FLASH_PRELOAD_ARGS(a) (a).tiles, (a).q, (a).kcache, (a).vcache, (a).ldq, (a).H, (a).KV, (a).max_ctx
#define QD_ROPE_PRELOAD_PARAMS                                                                     \
  bf16_t *qkv_, const int *row_pos_, const int *row_slot_, const float *q_gain_, const float *k_gain_, \
      const float2 *rope_, int ldqkv_, int H_
#define QD_ROPE_PRELOAD_SET(a) \
  do {                         \
    (a).qkv = qkv_;            \
    (a).row_pos = row_pos_;    \
    (a).row_slot = row_slot_;  \
    (a).q_gain = q_gain_;      \
    (a).k_gain = k_gain_;      \
    (a).rope = rope_;          \
    (a).ldqkv = ldqkv_;        \
    (a).H = H_;                \
  } while (0)
#define QD_ROPE_PRELOAD_ARGS(a) (a).qkv, (a).row_pos, (a).row_slot, (a).q_gain, (a).k_gain, (a).rope, (a).ldqkv, (a).H

// Leading scalar arguments of the batched projection kernels (k_skinny, k_skinny_norm,
// k_skinny_split, k_lm_skinny): the fields their first loads need, preloaded into SGPRs at
// wave launch, copied over the argument struct's (which is read from memory).
#define QD_SKINNY_PRELOAD_PARAMS                                                                \
  const int8_t *W_, const float *scale_, const bf16_t *x_, const int *x_rows_, const float *gain_, \
      int N_, int K_, int ldx_, int nb_
#define QD_SKINNY_PRELOAD_SET(a)                                                                  \
  do {                                                                                            \
    (a).W = W_;                                                                                   \
    (a).scale = scale_;                                                                           \
    (a).x = x_;                                                                                   \
    (a).x_rows = x_rows_;                                                                         \
    (a).gain = gain_;                                                                             \
    (a).N = N_;                                                                                   \
    (a).K = K_;                                                                                   \
    (a).ldx = ldx_;                                                                               \
    (a).nb = nb_;                                                                                 \
  } while (0)
#define QD_SKINNY_PRELOAD_ARGS(a) (a).W, (a).scale, (a).x, (a).x_rows, (a).gain, (a).N, (a).K, (a).ldx, (a).nb

// The fields the first loads need come as leading scalar arguments, which the hardware
// preloads into SGPRs at wave launch (the library is built with kernel-argument preloading);
// the rest are read from the argument segment in memory, off the first loads' path.  After the
// weights and scales, p0, p1, p2, i0, i1: the activation row, RMSNorm gains, row indices and
// row stride, or with MERGE the attention's split partials, their (max, sum) pairs, (unused),
// split count and head dim.
template <int R, int KC, int EPI, bool MERGE = false>
__global__ __launch_bounds__(256) void k_gemv1(const int8_t* W_, const float* scale_, const void* p0,
                                               const void* p1, const void* p2, int N_, int K_, int i0,
                                               int i1, GemvArgs a) {
  a.W = W_;
  a.scale = scale_;
  a.N = N_;
  a.K = K_;
  if constexpr (MERGE) {
    a.att_po = static_cast<const float*>(p0);
    a.att_ml = static_cast<const float*>(p1);
    a.att_ns = i0;
    a.att_D = i1;
  } else {
    a.x = static_cast<const bf16_t*>(p0);
    a.gain = static_cast<const float*>(p1);
    a.x_rows = static_cast<const int*>(p2);
    a.ldx = i0;
  }
  constexpr int NR = (EPI == EPI_SILU) ? 2 * R : R;  // weight rows per wave
  const int K = a.K;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nchunk = K >> 4;
  const int rows_per_blk = (EPI == EPI_SILU) ? 4 * R : 4 * R;  // logical outputs per block
  const int nout = (EPI == EPI_SILU) ? a.N / 2 : a.N;
  const int nblk = (nout + rows_per_blk - 1) / rows_per_blk;

  auto row_of = [&](int blk, int i) -> int {
    if (EPI == EPI_SILU) {
      const int j = blk * rows_per_blk + wid * R + (i % R);
      return j < nout ? gu_row(j, i / R) : a.N;
    }
    return blk * rows_per_blk + wid * R + i;
  };

  int blk = blockIdx.x;
  // Weights, scales, activations and gains are buffer loads whose out-of-range offset
  // reads zero, so no load sits in a branch: a load under a per-lane condition becomes an
  // exec-masked branch, and the compiler then waits for loads at the branch (one such wait
  // held back every later request until the first weight rows had arrived from HBM).
  constexpr int OOB = (int)0x80000000;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)a.scale, 0, a.N * 4, 0x00020000);
  // per-row scales (and residual values) of a block: requested with its weights, so the
  // epilogue after the reductions does not wait for another round trip
  // The residual values stay raw bf16 bits until the epilogue and are read from a clamped
  // (always valid) index: a conditional load converted in its branch would make the
  // wave wait for every load in flight, the weights included, at that point.
  float sc[NR];
  bf16_t rsb[R];
  auto load_rowdata = [&](int b) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = row_of(b, i);
      sc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            srs, (r < a.N && b < nblk) ? r * 4 : OOB, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int r = row_of(b, i);
      rsb[i] = EPI == EPI_RESID ? a.out[(r < a.N && b < nblk) ? r : 0] : (bf16_t)0;
    }
  };
  // weights of a block (rows r, 16-byte chunks ch of this lane)
  int4 wv[NR][KC];
  auto load_weights = [&](int b) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = row_of(b, i);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int ch = lane + 64 * c;
        wv[i][c] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(
                                                wrs, (r < a.N && ch < nchunk && b < nblk) ? r * K + ch * 16 : OOB, 0, 0));
      }
    }
  };
  // the activations and RMSNorm gains go out first, then the first block's weights and row
  // data: loads retire in order, so the norm waits only for its own inputs while the
  // weights are still in flight (the scheduling barrier keeps every request ahead of the
  // first use)
  const bf16_t* xrow = a.x + (size_t)(a.x_rows ? a.x_rows[0] : 0) * a.ldx;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc((void*)xrow, 0, K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t grs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.gain, 0, a.gain ? K * 4 : 0, 0x00020000);
  float xf[KC][16];
  float4 gq[KC][4];  // RMSNorm gains of this lane's chunks, requested with the activations
  uint4 xu[KC][2];
  if constexpr (MERGE) {
    // o = sum_s o_s 2^(m_s - m) / sum_s l_s 2^(m_s - m), m = max_s m_s, per head; splits in
    // ascending order, as the attention kernel's own merge adds them
    __shared__ __align__(16) bf16_t xm[64 * 16 * KC];
    constexpr int SM = ATT_DEFER_MAX_SPLITS;
    const int ns = a.att_ns, D = a.att_D, nh = K / D;
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.att_po, 0, nh * ns * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t mrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.att_ml, 0, nh * ns * 2 * 4, 0x00020000);
    struct MergeIn { float mv[SM], lv[SM]; float4 o0[SM], o1[SM]; };
    // every split's (max, sum) and 8 output dims of one head (d0 past K: all out of range)
    auto mload = [&](int d0, MergeIn& in) {
      const bool ok = d0 < K;
      const int h = ok ? d0 / D : 0, dd = ok ? d0 - h * D : 0;
#pragma unroll
      for (int s = 0; s < SM; ++s) {
        const bool sok = ok && s < ns;
        const int mo = (h * ns + s) * 8, po = ((h * ns + s) * D + dd) * 4;
        in.mv[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mrs, sok ? mo : OOB, 0, 0));
        in.lv[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mrs, sok ? mo + 4 : OOB, 0, 0));
        in.o0[s] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prs, sok ? po : OOB, 0, 0));
        in.o1[s] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prs, sok ? po + 16 : OOB, 0, 0));
      }
    };
    auto mstore = [&](int d0, const MergeIn& in) {
      float mx = -INFINITY;
#pragma unroll
      for (int s = 0; s < SM; ++s)
        if (s < ns) mx = fmaxf(mx, in.mv[s]);
      float lsum = 0.0f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < SM; ++s) {
        if (s >= ns || in.mv[s] == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(in.mv[s] - mx);
        lsum += in.lv[s] * w;
        const float ov[8] = {in.o0[s].x, in.o0[s].y, in.o0[s].z, in.o0[s].w,
                             in.o1[s].x, in.o1[s].y, in.o1[s].z, in.o1[s].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += ov[e] * w;
      }
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[e] = (uint32_t)f2bf(acc[2 * e] / lsum) | ((uint32_t)f2bf(acc[2 * e + 1] / lsum) << 16);
      *reinterpret_cast<uint4*>(&xm[d0]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    };
    // the thread's first 8 dims are requested before the weights (they come from L2 and
    // retire first), the weights and row data right behind them, then the merge
    {
      MergeIn in;
      mload(tid * 8, in);
      load_weights(blk);
      load_rowdata(blk);
      __builtin_amdgcn_sched_barrier(0);
      if (tid * 8 < K) mstore(tid * 8, in);
    }
    for (int d0 = tid * 8 + 256 * 8; d0 < K; d0 += 256 * 8) {  // rows wider than 2048
      MergeIn in;
      mload(d0, in);
      mstore(d0, in);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ch = lane + 64 * c;
      const bool cok = ch < nchunk;
      xu[c][0] = cok ? *reinterpret_cast<const uint4*>(&xm[ch * 16]) : make_uint4(0, 0, 0, 0);
      xu[c][1] = cok ? *reinterpret_cast<const uint4*>(&xm[ch * 16 + 8]) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) gq[c][q] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ch = lane + 64 * c;
      const bool cok = ch < nchunk;
      xu[c][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, cok ? ch * 32 : OOB, 0, 0));
      xu[c][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, cok ? ch * 32 + 16 : OOB, 0, 0));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        gq[c][q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  grs, cok ? ch * 64 + 16 * q : OOB, 0, 0));
    }
    load_weights(blk);
    load_rowdata(blk);
  }
  __builtin_amdgcn_sched_barrier(0);
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const uint4 u0 = xu[c][0], u1 = xu[c][1];
    const uint32_t w8[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xf[c][2 * j] = __uint_as_float(w8[j] << 16);
      xf[c][2 * j + 1] = __uint_as_float(w8[j] & 0xFFFF0000u);
      ss += xf[c][2 * j] * xf[c][2 * j] + xf[c][2 * j + 1] * xf[c][2 * j + 1];
    }
  }
  if (a.gain) {
    const float rinv = 1.0f / sqrtf(wave_sum(ss) / (float)K + a.eps);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nchunk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 g = gq[c][q];
          xf[c][4 * q + 0] = rbf(xf[c][4 * q + 0] * rinv * g.x);
          xf[c][4 * q + 1] = rbf(xf[c][4 * q + 1] * rinv * g.y);
          xf[c][4 * q + 2] = rbf(xf[c][4 * q + 2] * rinv * g.z);
          xf[c][4 * q + 3] = rbf(xf[c][4 * q + 3] * rinv * g.w);
        }
      }
    }
  }

  unsigned long long best = 0ull;
  for (; blk < nblk; blk += gridDim.x) {
    float acc[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      acc[i] = 0.0f;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        float wf[16];
        i8x16_to_f32(wv[i][c], wf);
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i] = fmaf(wf[j], xf[c][j], acc[i]);
      }
    }
    // next block's weights (and its scales, below) go out before the reductions
    const int nxt = blk + gridDim.x;
    float scn[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = row_of(nxt, i);
      scn[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             srs, (nxt < nblk && r < a.N) ? r * 4 : OOB, 0, 0));
    }
    if (nxt < nblk) load_weights(nxt);
#pragma unroll
    for (int i = 0; i < NR; ++i) acc[i] = wave_sum(acc[i]);
    if (lane == 0) {
      if (EPI == EPI_SILU) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int j = blk * rows_per_blk + wid * R + i;
          if (j >= nout) continue;
          const float g = rbf(acc[i] * sc[i]);
          const float u = rbf(acc[i + R] * sc[i + R]);
          a.out[j] = f2bf(g / (1.0f + expf(-g)) * u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int r = row_of(blk, i);
          if (r >= a.N) continue;
          const float v = acc[i] * sc[i];
          if (EPI == EPI_STORE) {
            a.out[r] = f2bf(v);
          } else if (EPI == EPI_RESID) {
            a.out[r] = f2bf(bf2f(rsb[i]) + rbf(v));
          } else {
            if (a.logits) a.logits[r] = v;
            const unsigned long long k = argmax_key(v, r);
            best = k > best ? k : best;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) sc[i] = scn[i];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int r = row_of(nxt, i);
      rsb[i] = EPI == EPI_RESID ? a.out[(nxt < nblk && r < a.N) ? r : 0] : (bf16_t)0;
    }
  }
  if (EPI == EPI_LOGITS) {
    __shared__ unsigned long long wbest[4];
    if (lane == 0) wbest[wid] = best;
    __syncthreads();
    unsigned long long b0 = 0ull;
    if (tid == 0) {
      b0 = wbest[0];
      for (int w = 1; w < 4; ++w) b0 = wbest[w] > b0 ? wbest[w] : b0;
    }
    lm_head_store(a, b0, 1);
  }
}

// ------------------------------------------------------------------------------------------
// prefill GEMM on MFMA: C[m][n] = scale[n] * sum_k A[m][k] * W[n][k]
// A bf16 [M][K], W int8 [N][K] converted to bf16 in registers (exact for |q| <= 127).
// 64x64 output tile per work-group, 4 waves in 2x2, each 32x32 = 2x2 MFMA 16x16x32 tiles.
// A buffer-load offset the compiler must hold in a register as computed (an empty asm
// statement that claims to change it): keeps a select between an in-range offset and the
// out-of-range one a select, instead of a branch around each load.
__device__ __forceinline__ int opaque_off(int off) {
  asm("" : "+v"(off));
  return off;
}

__device__ __forceinline__ bf16x8_t i8x8_to_bf16x8(uint2 w) {
  const uint32_t in[2] = {w.x, w.y};
  uint32_t out[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int v0 = ((int)(in[h] << (24 - 16 * e))) >> 24;
      const int v1 = ((int)(in[h] << (16 - 16 * e))) >> 24;
      // the upper halves of the two fp32 values (their exact bf16 forms) in one byte
      // permute: bytes 2, 3 of the first, then bytes 2, 3 of the second
      out[h * 2 + e] = __builtin_amdgcn_perm(__float_as_uint((float)v1), __float_as_uint((float)v0), 0x07060302u);
    }
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(out[0], out[1], out[2], out[3]));
}

// 64x64 output tile per work-group of 8 waves: k advances 128 per step, waves 0-3 take
// the first 64 k of each step and waves 4-7 the second (each group 2x2 waves of 32x32 =
// 2x2 MFMA 16x16x32 tiles), so every SIMD runs two independent chains between the
// step barriers; the two halves are added in LDS at the end.  The loads of GEMM_PF steps
// ahead are in flight while one step is multiplied out of LDS (double-buffered, one
// barrier per step); the weights are converted to bf16 once, when a step is written to
// LDS.  All loads are buffer loads whose out-of-range offsets read zero, so no load sits
// in a branch and each step waits only for its own data.  With split-K (blockIdx.z) each
// work-group stores its fp32 tile partial agent-coherently; the last of a tile's
// work-groups to arrive adds the partials in split order and runs the epilogue.
template <int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, int m, int n, float v, float vu,
                                              float sv, float su) {
  if (EPI == EPI_SILU) {
    const float g = rbf(v * sv);
    const float u = rbf(vu * su);
    const int j = (n / (2 * GU_BLOCK)) * GU_BLOCK + (n % GU_BLOCK);
    a.out[(size_t)m * a.ldo + j] = f2bf(g / (1.0f + expf(-g)) * u);
  } else {
    const float y = v * sv;
    bf16_t* o = a.out + (size_t)m * a.ldo + n;
    *o = (EPI == EPI_STORE) ? f2bf(y) : f2bf(bf2f(*o) + rbf(y));
  }
}

// Residual epilogue of a BM x BN tile through LDS: T (BM rows, pitch BN + 8) holds the
// tile's projections rounded to bf16, as the per-element epilogue rounds them; each of the
// NTH threads then updates 16-byte pieces of the residual rows, x = bf16(x + y), with all of
// its pieces' residual values requested at once, so the update costs one memory round trip
// where the per-element read-modify-write (each read waiting for the store before it) costs
// one per element.  N and ldo are multiples of 8 (the launcher checks).
template <int BM, int BN, int NTH>
__device__ __forceinline__ void resid_tile_update(const GemmArgs& a, const bf16_t* T, int m0, int n0) {
  constexpr int TP = BN + 8, PPR = BN / 8, NP = BM * PPR / NTH;
  static_assert(BM * PPR % NTH == 0, "whole passes");
  constexpr int OOB = (int)0x80000000;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t ors =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.out, 0, a.M * a.ldo * 2, 0x00020000);
  uint4 rv[NP];
  int off[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int idx = tid + NTH * u, row = idx / PPR, pc = idx % PPR;
    const int m = m0 + row, n = n0 + 8 * pc;
    off[u] = (m < a.M && n < a.N) ? (m * a.ldo + n) * 2 : OOB;
    rv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ors, off[u], 0, 0));
  }
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int idx = tid + NTH * u, row = idx / PPR, pc = idx % PPR;
    const uint4 y = *reinterpret_cast<const uint4*>(&T[row * TP + 8 * pc]);
    const uint32_t xw[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w}, yw[4] = {y.x, y.y, y.z, y.w};
    uint32_t ow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(xw[e] << 16) + __uint_as_float(yw[e] << 16);
      const float hi = __uint_as_float(xw[e] & 0xFFFF0000u) + __uint_as_float(yw[e] & 0xFFFF0000u);
      ow[e] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
    }
    if (off[u] != OOB)
      *reinterpret_cast<uint4*>(a.out + (size_t)(m0 + row) * a.ldo + n0 + 8 * pc) =
          make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

constexpr int GEMM_PF = 4;  // k-steps of loads in flight
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int EPI>
__global__ __launch_bounds__(512) void k_gemm(QD_GEMM_PRELOAD_PARAMS, GemmArgs a) {
  QD_GEMM_PRELOAD_SET(a);
  constexpr int BM = 64, BN = 64, BK = 128, P = GEMM_PF;
  constexpr int OOB = (int)0x80000000;
  // LDS holds each 16-row x 32-k operand fragment in MFMA lane order (lane l's 8 values in
  // 16-byte slot l ^ ((l / 16) % 4) of a 1088-byte fragment slot), so a fragment read is
  // 1 KB of consecutive bytes
  constexpr int FRAG = 1088;
  constexpr int NFRAG = (BM / 16) * (BK / 32);  // 16 fragments per operand per stage
  __shared__ __align__(16) unsigned char Ab[2][NFRAG * FRAG];
  __shared__ __align__(16) unsigned char Wb[2][NFRAG * FRAG];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kh = wid >> 2, wm = wid & 1, wn = (wid >> 1) & 1;
  const int grp = lane >> 4, r16 = lane & 15;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int S = a.splits, z = blockIdx.z;
  const int kper = ((a.K + S - 1) / S + 31) & ~31;
  const int kbeg = z * kper;
  const int kend = min(a.K, kbeg + kper);
  const int nsteps = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  // rows past M (N) lie past the end of A (W) and read zero; k past the split's end is
  // sent out of range explicitly
  const __amdgpu_buffer_rsrc_t arsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, a.M * a.lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * a.K, 0x00020000);
  // staging: thread j = tid%8 of row tid/8 brings k 16j .. 16j+15 of the step for both A
  // and W.  Within a step, k = 16j + e sits in 8-value chunk j (e < 8) or 8 + j (e >= 8),
  // the same permutation for both operands, so the dot products are unchanged.
  const int sr = tid >> 3, sj = tid & 7, sw = sj * 16;
  auto slot = [](int row, int c) {  // byte offset of 8-value chunk c (of 16) of stage row row
    const int pos = (row & 15) + 16 * (c & 3);
    return ((row >> 4) * 4 + (c >> 2)) * FRAG + 16 * (pos ^ (c & 3));
  };
  struct Stage { uint4 a0, a1, w; };
  auto fetch = [&](int step, Stage& q) {
    const int k = kbeg + step * BK;
    const int abase = ((m0 + sr) * a.lda + k + sw) * 2;
    q.a0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(arsc, k + sw < kend ? abase : OOB, 0, 0));
    q.a1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         arsc, k + sw + 8 < kend ? abase + 16 : OOB, 0, 0));
    q.w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                        wrsc, k + sw < kend ? (n0 + sr) * a.K + k + sw : OOB, 0, 0));
  };
  auto stash = [&](const Stage& q, int buf) {
    *reinterpret_cast<uint4*>(&Ab[buf][slot(sr, sj)]) = q.a0;
    *reinterpret_cast<uint4*>(&Ab[buf][slot(sr, 8 + sj)]) = q.a1;
    *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(sr, sj)]) = i8x8_to_bf16x8(make_uint2(q.w.x, q.w.y));
    *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(sr, 8 + sj)]) = i8x8_to_bf16x8(make_uint2(q.w.z, q.w.w));
  };
  const int rd = 16 * (lane ^ (grp & 3));  // this lane's slot in every fragment read

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // scales of this lane's two output channels (gate/up: the pair), requested first
  float gsc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + wn * 32 + nt * 16 + r16;
    gsc[nt] = a.scale[n < a.N ? n : 0];
  }

  Stage q[P];
#pragma unroll
  for (int u = 0; u < P; ++u) fetch(u, q[u]);
  // residual inputs of this lane's 16 outputs, requested behind the first steps' loads as
  // raw bits from in-range offsets (out-of-range reads zero), so no wait lands in a branch
  uint32_t res[2][4][2];
  if constexpr (EPI == EPI_RESID) {
    const __amdgpu_buffer_rsrc_t orsc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.out, 0, a.M * a.ldo * 2, 0x00020000);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int m = m0 + wm * 32 + mt * 16 + 4 * grp + i;
          const int n = n0 + wn * 32 + nt * 16 + r16;
          res[mt][i][nt] = __builtin_amdgcn_raw_buffer_load_b16(
              orsc, (m < a.M && n < a.N) ? (m * a.ldo + n) * 2 : OOB, 0, 0);
        }
  }
  stash(q[0], 0);
  __syncthreads();
  // whole groups of P steps (steps past the end multiply zeros): an early exit from the
  // unrolled group would leave different loads pending on each path, and the wait at the
  // loop head would then drain all of them
  for (int i0 = 0; i0 < nsteps; i0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int i = i0 + u;
      const int buf = i & 1;
      fetch(i + P, q[u]);  // into the slot step i vacated
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int kf = kh * 2 + sub;  // 32-k fragment of the step
        bf16x8_t af[2], bw[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          af[mt] = *reinterpret_cast<const bf16x8_t*>(&Ab[buf][((wm * 2 + mt) * 4 + kf) * FRAG + rd]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bw[nt] = *reinterpret_cast<const bf16x8_t*>(&Wb[buf][((wn * 2 + nt) * 4 + kf) * FRAG + rd]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bw[nt], acc[mt][nt], 0, 0, 0);
      }
      stash(q[u + 1 < P ? u + 1 : 0], buf ^ 1);  // step i + 1 (zeros past the end)
      __syncthreads();
    }
  }
  // the second k half joins the first through LDS (the staging buffers are free now);
  // waves 0-3 continue with the sum
  float* red = reinterpret_cast<float*>(&Ab[0][0]);  // [4 waves][16][64] floats
  if (kh == 1) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wid - 4) * 16 + (mt * 2 + nt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
  }
  __syncthreads();
  const bool lead = kh == 0;  // waves 4-7 stay for the barriers below but do no more work
  if (lead) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][nt][i] += red[(wid * 16 + (mt * 2 + nt) * 4 + i) * 64 + lane];
  }

  if constexpr (EPI == EPI_PART) {
    // this split's fp32 partial of the lane's 16 outputs, [z][M][N]; merged downstream
    if (!lead) return;
    float* pz = a.part + (size_t)z * a.M * a.N;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 32 + mt * 16 + 4 * grp + i;
        if (m >= a.M) continue;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = n0 + wn * 32 + nt * 16 + r16;
          if (n < a.N) pz[(size_t)m * a.N + n] = acc[mt][nt][i];
        }
      }
    return;
  }
  if (S > 1) {
    // tile partial, thread-major: 16 floats of lead thread tid at ((tile * S + z) * 256 + tid) * 16
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (size_t)tile * S * 4096, 0, S * 4096 * 4, 0x00020000);
    if (lead) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[mt][nt]), prs,
                                                 ((z * 256 + tid) * 16 + (mt * 2 + nt) * 4) * 4, 0, 16);
    }
    // every store of this work-group has completed before thread 0 counts it in
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      is_last = __hip_atomic_fetch_add(a.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (unsigned)(S - 1);
    __syncthreads();
    if (!is_last || !lead) return;
    f32x4_t tot[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) tot[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 4) {
      f32x4_t pv[4][2][2];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int sj = s0 + j;
            const int off = (sj < S && sj != z) ? ((sj * 256 + tid) * 16 + (mt * 2 + nt) * 4) * 4 : OOB;
            pv[j][mt][nt] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 16));
          }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int sj = s0 + j;
            if (sj < S) tot[mt][nt] += sj == z ? acc[mt][nt] : pv[j][mt][nt];
          }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = tot[mt][nt];
    if (tid == 0) __hip_atomic_store(a.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!lead) return;

  // lane holds D[4*(lane/16)+i][lane%16]: token rows, channel columns
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 32 + mt * 16 + 4 * grp + i;
      if (m >= a.M) continue;
      if (EPI == EPI_SILU) {
        const int ng = n0 + wn * 32 + r16;
        if (ng + GU_BLOCK < a.N)
          gemm_epilogue<EPI_SILU>(a, m, ng, acc[mt][0][i], acc[mt][1][i], gsc[0], gsc[1]);
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = n0 + wn * 32 + nt * 16 + r16;
          if (n >= a.N) continue;
          const float y = acc[mt][nt][i] * gsc[nt];
          a.out[(size_t)m * a.ldo + n] =
              EPI == EPI_RESID ? f2bf(bf2f((bf16_t)res[mt][i][nt]) + rbf(y)) : f2bf(y);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Prefill GEMM for few token rows (up to 128): a 64x64 output tile per work-group of
// 8 waves, each wave a 32*C-wide k slice of it (k-split z of the grid covers 256*C of K).
// Every wave requests all of its operand fragments at once, straight into MFMA operand
// registers (A: 16 bytes of 8 bf16 per lane and fragment; W: 8 int8 codes, converted
// exactly to bf16 in registers), multiplies its slice, and the 8 partial tiles are added
// once through LDS.  There is no per-k-step barrier or LDS staging: the tile's latency is
// one memory round trip, its MFMAs and one reduction, where the k-stepped kernel walks a
// serial chain of K/128 steps.  128 KB of LDS: one work-group per CU.
template <int EPI, int C>
__global__ __launch_bounds__(512) void k_gemm_ks(QD_GEMM_PRELOAD_PARAMS, GemmArgs a) {
  QD_GEMM_PRELOAD_SET(a);
  constexpr int OOB = (int)0x80000000;
  __shared__ __align__(16) f32x4_t red[8][16][64];  // [wave][m tile * 4 + n tile][lane]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = lane >> 4, r16 = lane & 15;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64, z = blockIdx.z;
  const int k0 = z * (256 * C) + wid * (32 * C);
  const __amdgpu_buffer_rsrc_t arsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, a.M * a.lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * a.K, 0x00020000);
  // fragment (tile t, chunk c): lane holds row 16t + lane%16, k = k0 + 32c + 8*(lane/16) .. +8;
  // rows past M (N) and k past K read zero
  uint4 af[4][C];
  uint2 wf[4][C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int k = k0 + 32 * c + 8 * grp;
    const bool ok = k < a.K;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      af[t][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               arsc, ok ? ((m0 + 16 * t + r16) * a.lda + k) * 2 : OOB, 0, 0));
#pragma unroll
    for (int t = 0; t < 4; ++t)
      wf[t][c] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                               wrsc, ok ? (n0 + 16 * t + r16) * a.K + k : OOB, 0, 0));
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bf16x8_t bw = i8x8_to_bf16x8(wf[nt][c]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[mt][c]),
                                                              bw, acc[mt][nt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) red[wid][mt * 4 + nt][lane] = acc[mt][nt];
  __syncthreads();
  // the 8 slices of each of the 16 x 64 lane positions, added in wave order; a position
  // (tile mt*4+nt, lane ln) holds D[m0 + 16mt + 4(ln/16) + i][n0 + 16nt + ln%16], i < 4
  auto sum8 = [&](int t, int ln) {
    f32x4_t v = red[0][t][ln];
#pragma unroll
    for (int w = 1; w < 8; ++w) v += red[w][t][ln];
    return v;
  };
  if constexpr (EPI == EPI_SILU) {
    // thread: m tile, gate/up pair, lane position -> the gate (n tile 2p) and up (2p+1) sums
    const int mt = tid >> 7, pr = (tid >> 6) & 1, ln = tid & 63;
    const f32x4_t g = sum8(mt * 4 + 2 * pr, ln), u = sum8(mt * 4 + 2 * pr + 1, ln);
    const int ng = n0 + 32 * pr + (ln & 15);
    const float sg = a.scale[ng < a.N ? ng : 0], su = a.scale[ng + GU_BLOCK < a.N ? ng + GU_BLOCK : 0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * mt + 4 * (ln >> 4) + i;
      if (m < a.M && ng + GU_BLOCK < a.N) gemm_epilogue<EPI_SILU>(a, m, ng, g[i], u[i], sg, su);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + 512 * j, t = idx >> 6, ln = idx & 63;
      const int mt = t >> 2, nt = t & 3;
      const f32x4_t v = sum8(t, ln);
      const int n = n0 + 16 * nt + (ln & 15);
      if (n >= a.N) continue;
      if constexpr (EPI == EPI_PART) {
        float* pz = a.part + (size_t)z * a.M * a.N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * mt + 4 * (ln >> 4) + i;
          if (m < a.M) pz[(size_t)m * a.N + n] = v[i];
        }
      } else {
        const float sc = a.scale[n];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * mt + 4 * (ln >> 4) + i;
          if (m < a.M) gemm_epilogue<EPI>(a, m, n, v[i], 0.0f, sc, 0.0f);
        }
      }
    }
  }
}

// Sum of v over an aligned group of L = 8 or 16 lanes in the order of a butterfly over the
// lane index (lane ^ 1, then lane ^ 2, ..: every lane adds its partner's partial to its
// own), with DPP lane moves in place of LDS permutes: after the first two levels the four
// lanes of a quad hold equal values, so the half-row mirror (lane 7 - i) brings lane i the
// other quad's sum exactly as lane ^ 4 would, and the row mirror (lane 15 - i) the other
// eight lanes' sum as lane ^ 8 would.
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(L == 8 || L == 16, "8 or 16 lanes");
  if constexpr (L == 16) return row16_sum(v);
  v += dpp_f<0xB1>(0.0f, v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(0.0f, v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(0.0f, v);  // row_half_mirror
  return v;
}

// One (row, head) item of the q|k|v epilogue below, dims 4j .. 4j+3 and D/2+4j .. of lane j
// (the head's L = D/8 lanes are consecutive): the head's sum of squares across those lanes,
// then the q / K RMSNorm and RoPE at the row's position (slot sl, position p, factors
// c01 = (cos, sin) of dims 4j, 4j+1 and c23 of 4j+2, 4j+3), or the V copy.  Every lane
// takes part in the sum, also for rows past M.  D is 64 or 128.
template <int D>
__device__ __forceinline__ void rope_item(const GemmArgs& a, const bf16_t* T, int TP, int row, int hl, int m0,
                                          int n0, int j, int sl, int p, float4 c01, float4 c23, float4 gq1,
                                          float4 gq2, float4 gk1, float4 gk2) {
  const RopeArgs& r = a.rope;
  constexpr int half = D >> 1, L = D >> 3;
  const int nheads = r.H + 2 * r.KV;
  const int m = m0 + row, hh = n0 / D + hl;
  const int c0 = row * TP + hl * D + 4 * j;
  const uint2 u1 = *reinterpret_cast<const uint2*>(&T[c0]);
  const uint2 u2 = *reinterpret_cast<const uint2*>(&T[c0 + half]);
  const uint32_t w1[2] = {u1.x, u1.y}, w2[2] = {u2.x, u2.y};
  float x1[4], x2[4], ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    x1[2 * e] = __uint_as_float(w1[e] << 16);
    x1[2 * e + 1] = __uint_as_float(w1[e] & 0xFFFF0000u);
    x2[2 * e] = __uint_as_float(w2[e] << 16);
    x2[2 * e + 1] = __uint_as_float(w2[e] & 0xFFFF0000u);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
  ss = lane_group_sum<L>(ss);
  if (m >= r.M || hh >= nheads) return;
  if (hh >= r.H + r.KV) {
    bf16_t* dst = r.vcache + (((size_t)sl * r.KV + (hh - r.H - r.KV)) * r.max_ctx + p) * D;
    *reinterpret_cast<uint2*>(dst + 4 * j) = u1;
    *reinterpret_cast<uint2*>(dst + half + 4 * j) = u2;
    return;
  }
  const bool isq = hh < r.H;
  const float4 g1 = isq ? gq1 : gk1, g2 = isq ? gq2 : gk2;
  const float gv1[4] = {g1.x, g1.y, g1.z, g1.w}, gv2[4] = {g2.x, g2.y, g2.z, g2.w};
  const float cv[4] = {c01.x, c01.z, c23.x, c23.z}, sv[4] = {c01.y, c01.w, c23.y, c23.w};
  const float rinv = 1.0f / sqrtf(ss / (float)D + r.eps);
  // (bf16 roundings two at a time: one conversion instruction per pair of values)
  auto bf2 = [](float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
  };
  uint32_t o1[2], o2[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int q0 = 2 * e, q1 = 2 * e + 1;
    const uint32_t yb1 = bf2(x1[q0] * rinv * gv1[q0], x1[q1] * rinv * gv1[q1]);
    const uint32_t yb2 = bf2(x2[q0] * rinv * gv2[q0], x2[q1] * rinv * gv2[q1]);
    const float y1a = __uint_as_float(yb1 << 16), y1b = __uint_as_float(yb1 & 0xFFFF0000u);
    const float y2a = __uint_as_float(yb2 << 16), y2b = __uint_as_float(yb2 & 0xFFFF0000u);
    o1[e] = bf2(y1a * cv[q0] - y2a * sv[q0], y1b * cv[q1] - y2b * sv[q1]);
    o2[e] = bf2(y2a * cv[q0] + y1a * sv[q0], y2b * cv[q1] + y1b * sv[q1]);
  }
  bf16_t* dst = isq ? a.out + (size_t)m * a.ldo + (size_t)hh * D
                    : r.kcache + (((size_t)sl * r.KV + (hh - r.H)) * r.max_ctx + p) * D;
  *reinterpret_cast<uint2*>(dst + 4 * j) = make_uint2(o1[0], o1[1]);
  *reinterpret_cast<uint2*>(dst + half + 4 * j) = make_uint2(o2[0], o2[1]);
}

// ------------------------------------------------------------------------------------------
// Epilogue of a q|k|v projection tile with the QK-norm, RoPE and K/V cache writes fused in
// (head dim D = 64 or 128, so no head straddles two tiles).  The tile's projections,
// rounded to bf16 as the plain store would write them, are in LDS (T: BM rows, pitch BN + 8
// elements, over the stage buffers once every stage read has passed a barrier); then D/8
// lanes take one (row, head): dims 4j..4j+3 and D/2+4j..D/2+4j+3 of lane j, the sum of
// squares over the head added across those lanes, the RMSNorm with the head's shared gain
// and the rotate-half rotation at the row's position as k_qk_rope computes them.  q heads
// are written back to the projection's output, K heads to the K cache at (slot, position)
// of the row, V heads copied to the V cache.  NT threads; D (64 or 128) equals rope.D.
template <int BM, int BN, int NT, int D>
__device__ __forceinline__ void gemm_rope_tile(const GemmArgs& a, const bf16_t* T, int m0, int n0) {
  constexpr int TP = BN + 8;
  constexpr int NIT = BM * BN / 8 / NT;  // (row, head, lane part) items per thread
  const int tid = threadIdx.x;
  const RopeArgs& r = a.rope;
  constexpr int half = D >> 1, L = D >> 3, lgL = __builtin_ctz(L);
  constexpr int hpt = BN / D;
  // item it of this thread: idx = it * NT + tid, its dims 4j .. and D/2 + 4j .. with
  // j = tid % L the same for every item (NT is a multiple of L), so the thread's q and k
  // gains are loaded once.  Every item's row slot and position are requested together and
  // waited for once, then the RoPE factors group by group, each group's before its stores:
  // stores count with loads, so a load issued among stores would wait for them.
  const int j = tid & (L - 1);
  const float4 gq1 = *reinterpret_cast<const float4*>(r.q_gain + 4 * j);
  const float4 gq2 = *reinterpret_cast<const float4*>(r.q_gain + half + 4 * j);
  const float4 gk1 = *reinterpret_cast<const float4*>(r.k_gain + 4 * j);
  const float4 gk2 = *reinterpret_cast<const float4*>(r.k_gain + half + 4 * j);
  int slot[NIT], pos[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int gi = (it * NT + tid) >> lgL;
    const int m = m0 + gi / hpt;
    const int mc = m < r.M ? m : r.M - 1;
    slot[it] = r.row_slot[mc];
    pos[it] = r.row_pos[mc];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
  // the items in groups of NG (registers for every item's RoPE factors at once would spill):
  // a group's factors are requested together, then its stores go out
  constexpr int NG = NIT > 8 ? 8 : NIT;
  static_assert(NIT % NG == 0, "whole groups");
#pragma unroll
  for (int g0 = 0; g0 < NIT; g0 += NG) {
    float4 c01[NG], c23[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float2* rp = r.rope + (size_t)pos[g0 + k] * half + 4 * j;  // (cos, sin) of dims 4j ..
      c01[k] = *reinterpret_cast<const float4*>(rp);
      c23[k] = *reinterpret_cast<const float4*>(rp + 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: the group's factors (and earlier stores)
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int gi = ((g0 + k) * NT + tid) >> lgL;
      const int row = gi / hpt;
      rope_item<D>(a, T, TP, row, gi - row * hpt, m0, n0, j, slot[g0 + k], pos[g0 + k], c01[k], c23[k], gq1, gq2,
                gk1, gk2);
    }
  }
}

// the 128x128-tile kernel's accumulators (4 waves of 64x64) into T, then the epilogue
__device__ __forceinline__ void gemm_big_rope_epilogue(const GemmArgs& a, bf16_t* T,
                                                       const f32x4_t (&acc)[4][4], const float (&gsc)[4],
                                                       int m0, int n0, int wm, int wn) {
  constexpr int TP = 136;
  const int lane = threadIdx.x & 63, grp = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        T[(wm * 64 + mt * 16 + 4 * grp + i) * TP + wn * 64 + nt * 16 + r16] = f2bf(acc[mt][nt][i] * gsc[nt]);
  __syncthreads();
  if (a.rope.D == 128) gemm_rope_tile<128, 128, 256, 128>(a, T, m0, n0);
  else gemm_rope_tile<128, 128, 256, 64>(a, T, m0, n0);
}

// q|k|v projection at a few hundred token rows with the QK-norm, RoPE and K/V cache writes
// in its epilogue: 32x128 output tiles (a 128-wide tile holds whole heads, so the epilogue
// needs no other tile's outputs), the same 4096 outputs and 8 waves per work-group as the
// 64x64 kernel above, so a 256-row prompt still gives every CU a tile.  k advances 128 per
// step; waves 0-3 take the first 64 k of each step and waves 4-7 the second, each wave a
// 32x32 block of 2x2 MFMA 16x16x32 tiles, the halves added in LDS at the end.  GEMM_PF
// steps of loads in flight, double-buffered LDS, one barrier per step, the weights turned
// into bf16 when a step is written to LDS.  Staging: A row t / 16 takes k 8 (t % 16) ..
// of the step from thread t, W row t / 4 takes k 32 (t % 4) .. (two 16-byte loads), both
// in natural k order.  No split-K: one work-group per tile.
__global__ __launch_bounds__(512) void k_gemm_qr(QD_GEMM_PRELOAD_PARAMS, GemmArgs a) {
  QD_GEMM_PRELOAD_SET(a);
  constexpr int BM = 32, BN = 128, BK = 128, P = GEMM_PF;
  constexpr int OOB = (int)0x80000000;
  constexpr int FRAG = 1088;  // one 16-row x 32-k fragment in MFMA lane order (+ padding)
  constexpr int AFR = (BM / 16) * (BK / 32), WFR = (BN / 16) * (BK / 32);
  __shared__ __align__(16) unsigned char Ab[2][AFR * FRAG];
  __shared__ __align__(16) unsigned char Wb[2][WFR * FRAG];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int kh = wid >> 2, wn = wid & 3;
  const int grp = lane >> 4, r16 = lane & 15;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int K = a.K;
  const int nsteps = (K + BK - 1) / BK;

  // rows past M (N) lie past the end of A (W) and read zero; k past K is sent out of range
  const __amdgpu_buffer_rsrc_t arsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, a.M * a.lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * K, 0x00020000);
  const int ar = tid >> 4, ac = tid & 15;  // A: row, 8-value chunk
  const int wr = tid >> 2, wq = tid & 3;   // W: row, 32-value quarter
  auto slot = [](int row, int c) {  // byte offset of 8-value chunk c (of 16) of stage row row
    const int pos = (row & 15) + 16 * (c & 3);
    return ((row >> 4) * 4 + (c >> 2)) * FRAG + 16 * (pos ^ (c & 3));
  };
  struct Stage { uint4 a, w0, w1; };
  auto fetch = [&](int step, Stage& q) {
    const int k = step * BK;
    q.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                        arsc, k + 8 * ac < K ? ((m0 + ar) * a.lda + k + 8 * ac) * 2 : OOB, 0, 0));
    const int wo = (n0 + wr) * K + k + 32 * wq;
    q.w0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsc, k + 32 * wq < K ? wo : OOB, 0, 0));
    q.w1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         wrsc, k + 32 * wq + 16 < K ? wo + 16 : OOB, 0, 0));
  };
  auto stash = [&](const Stage& q, int buf) {
    *reinterpret_cast<uint4*>(&Ab[buf][slot(ar, ac)]) = q.a;
    *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(wr, 4 * wq)]) = i8x8_to_bf16x8(make_uint2(q.w0.x, q.w0.y));
    *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(wr, 4 * wq + 1)]) = i8x8_to_bf16x8(make_uint2(q.w0.z, q.w0.w));
    *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(wr, 4 * wq + 2)]) = i8x8_to_bf16x8(make_uint2(q.w1.x, q.w1.y));
    *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(wr, 4 * wq + 3)]) = i8x8_to_bf16x8(make_uint2(q.w1.z, q.w1.w));
  };
  const int rd = 16 * (lane ^ (grp & 3));  // this lane's slot in every fragment read

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float gsc[2];  // scales of this lane's two output channels, requested first
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + wn * 32 + nt * 16 + r16;
    gsc[nt] = a.scale[n < a.N ? n : 0];
  }

  // the epilogue's inputs, requested ahead of the k loop.  One (row, head) item per thread
  // (32 rows x 128 columns in parts of 8 dims): row and head from tid / (D/8), dims 4j ..
  // and D/2 + 4j .. with j = tid % (D/8).  Its row's slot and position, the q and k gains of
  // its dims (the RoPE factors at its position follow the k loop)
  const RopeArgs& r = a.rope;
  const int L = r.D >> 3, half = r.D >> 1, hpt = BN / r.D;
  const int rj = tid & (L - 1), rgi = tid >> __builtin_ctz(L), rrow = rgi / hpt;
  const int rmc = min(m0 + rrow, a.M - 1);
  const int rsl = r.row_slot[rmc], rpos = r.row_pos[rmc];
  const float4 gq1 = *reinterpret_cast<const float4*>(r.q_gain + 4 * rj);
  const float4 gq2 = *reinterpret_cast<const float4*>(r.q_gain + half + 4 * rj);
  const float4 gk1 = *reinterpret_cast<const float4*>(r.k_gain + 4 * rj);
  const float4 gk2 = *reinterpret_cast<const float4*>(r.k_gain + half + 4 * rj);

  Stage q[P];
#pragma unroll
  for (int u = 0; u < P; ++u) fetch(u, q[u]);
  stash(q[0], 0);
  __syncthreads();
  // whole groups of P steps (steps past the end multiply zeros), as in the 64x64 kernel
  for (int i0 = 0; i0 < nsteps; i0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int i = i0 + u;
      const int buf = i & 1;
      fetch(i + P, q[u]);  // into the slot step i vacated
      // (the next step's conversion stays behind this step's MFMAs, so its wait counts the
      // loads issued since)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int kf = kh * 2 + sub;  // 32-k fragment of the step
        bf16x8_t af[2], bw[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          af[mt] = *reinterpret_cast<const bf16x8_t*>(&Ab[buf][(mt * 4 + kf) * FRAG + rd]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bw[nt] = *reinterpret_cast<const bf16x8_t*>(&Wb[buf][((wn * 2 + nt) * 4 + kf) * FRAG + rd]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bw[nt], acc[mt][nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      stash(q[u + 1 < P ? u + 1 : 0], buf ^ 1);  // step i + 1 (zeros past the end)
      __syncthreads();
    }
  }
  // the RoPE factors of the epilogue's item ((cos, sin) of dims 4j ..), in flight while the
  // k halves are added
  const float2* rp = r.rope + (size_t)rpos * half + 4 * rj;
  const float4 c01 = *reinterpret_cast<const float4*>(rp);
  const float4 c23 = *reinterpret_cast<const float4*>(rp + 2);
  // the second k half joins the first through LDS (the staging buffers are free now)
  float* red = reinterpret_cast<float*>(&Wb[0][0]);  // [4 waves][16][64] floats
  if (kh == 1) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wid - 4) * 16 + (mt * 2 + nt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
  }
  __syncthreads();
  // the tile's projections, rounded to bf16 as the plain store would write them, into T
  // (32 rows, pitch 136) for the QK-norm / RoPE epilogue
  bf16_t* T = reinterpret_cast<bf16_t*>(&Ab[0][0]);
  constexpr int TP = BN + 8;
  if (kh == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          T[(mt * 16 + 4 * grp + i) * TP + wn * 32 + nt * 16 + r16] =
              f2bf((acc[mt][nt][i] + red[(wid * 16 + (mt * 2 + nt) * 4 + i) * 64 + lane]) * gsc[nt]);
  }
  __syncthreads();
  if (r.D == 128) rope_item<128>(a, T, TP, rrow, rgi - rrow * hpt, m0, n0, rj, rsl, rpos, c01, c23, gq1, gq2, gk1, gk2);
  else rope_item<64>(a, T, TP, rrow, rgi - rrow * hpt, m0, n0, rj, rsl, rpos, c01, c23, gq1, gq2, gk1, gk2);
}

// Prefill GEMM for the widest projections at many token rows, operands loaded straight
// into LDS (global_load_lds: lane i of a load writes LDS base + 16 i), so no staging
// registers are needed and 8 waves (two per SIMD) each hold a 128x64 block of 8x4 MFMA
// 16x16x32 tiles of the 256x256 output tile: every A fragment read feeds four MFMAs, every
// W fragment eight.  Three 64-k stages rotate through 144 KB of LDS; a stage's loads are
// issued in the middle of the stage three before it.  A rows (128 bytes of a stage) keep their 16-byte chunks XOR-
// swizzled by row (chunk c at slot c ^ ((row / 2) % 8)) and W rows (64 int8 bytes) theirs
// by (row / 4) % 4, so the loads read whole row segments and the 16 consecutive lanes of a
// fragment read (16 rows) hit 16 different 16-byte bank groups of the 64 banks.  The weights stay int8 in LDS: a lane reads 16 codes
// (k 16g .. 16g + 15 of the stage) and converts them for both 32-k halves; the A chunks
// follow the same k order (half h of lane group g: k 16g + 8h ..).
constexpr int DL_STAGES = 3;
// 16 bytes per lane from global memory (a wave-uniform base address plus this lane's 32-bit
// byte offset) to LDS at m0 + 16 * lane (m0 = lds_base, uniform over the wave).  Issued from
// inline assembly so that the compiler does not order later LDS reads behind it: it does not
// know these writes, and the kernel waits for them itself (the load has no register result;
// its address registers are read at issue).
__device__ __forceinline__ void lds_dma16_s(const void* base, unsigned off, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_base)
               : "memory", "m0");
}
// WM = 2: 256x256 tiles, waves 2 (rows) x 4 (channels) of 128x64; WM = 4: 256x128 tiles for
// the narrow projections (O and down), waves 4 x 2 of 64x64.
template <int EPI, int WM>
__global__ __launch_bounds__(512, 1) void k_gemm_dl(QD_GEMM_PRELOAD_PARAMS, GemmArgs a) {
  QD_GEMM_PRELOAD_SET(a);
  constexpr int WN = 8 / WM, MT = 16 / WM;  // waves along channels, 16-row tiles per wave
  constexpr int BM = 256, BN = 64 * WN, BK = 64;
  constexpr int A_BYTES = BM * BK * 2, W_BYTES = BN * BK;  // 32 KB + 16 (8) KB per stage
  constexpr int WL = BN / 128;                             // W loads per wave and stage
  // stage b: A at b * A_BYTES, W at 3 * A_BYTES + b * W_BYTES; the q|k|v epilogue reuses the
  // first 256 x 264 bf16 (135 KB) as its tile
  __shared__ __align__(16) unsigned char lds[DL_STAGES * (A_BYTES + W_BYTES)];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WM, wn = wid / WM;
  const int grp = lane >> 4, r16 = lane & 15;
  const int ntn = (a.N + BN - 1) / BN, ntm = (a.M + BM - 1) / BM, ntiles = ntn * ntm;
  const int q8 = ntiles >> 3, r8 = ntiles & 7, xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int t = xcd * q8 + min(xcd, r8) + loc;
  const int m0 = (t / ntn) * BM, n0 = (t % ntn) * BN;
  const int nsteps = (a.K + BK - 1) / BK;
  // this lane's loads: A load j (of 4) covers stage rows 8 * (4 * wid + j) .. +8 (1 KB);
  // lane -> row r = 8 * (4 * wid + j) + lane / 8, LDS slot lane % 8, holding chunk
  // (lane % 8) ^ ((r / 2) % 8); W load j (of WL) covers rows 16 * (WL * wid + j) .. +16;
  // lane -> row 16 * (WL * wid + j) + lane / 4, slot lane % 4, holding chunk
  // (lane % 4) ^ ((r / 4) % 4).
  // Rows past M (N) read row 0 of the operand (their outputs are never stored); k past K
  // is never requested (K is a multiple of 64 here).
  // (byte offsets from the operand bases; the launch checks that they fit 31 bits)
  unsigned ag[4], wg[WL];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * (4 * wid + j) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int m = m0 + r < a.M ? m0 + r : 0;
    ag[j] = (unsigned)(m * a.lda + 8 * c) * 2u;
  }
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    const int r = 16 * (WL * wid + j) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int n = n0 + r < a.N ? n0 + r : 0;
    wg[j] = (unsigned)(n * a.K + 16 * c);
  }
  // stage buffers by compile-time index
  auto issue = [&](auto bc, int step) {
    constexpr int b = decltype(bc)::value;
    unsigned char* Ad = lds + b * A_BYTES;
    unsigned char* Wd = lds + DL_STAGES * A_BYTES + b * W_BYTES;
    const int k0 = step * BK;
    const unsigned ab = __builtin_amdgcn_readfirstlane((unsigned)(size_t)Ad + 4096u * wid);
    const unsigned wb = __builtin_amdgcn_readfirstlane((unsigned)(size_t)Wd + 1024u * WL * wid);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_dma16_s(a.A + k0, ag[j], ab + 1024u * j);
#pragma unroll
    for (int j = 0; j < WL; ++j) lds_dma16_s(a.W + k0, wg[j], wb + 1024u * j);
  };
  // fragment reads: A fragment f (rows 16f .. +16), half h: lane (r16, g) reads chunk
  // 2g + h of row 16f + r16; W fragment f: lane reads chunk g of row 16f + r16
  f32x4_t acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over the 64-k stages (buffer b = stage % 3).  A stage's W chunks and
  // first A half are read before its MFMAs start; its second A half is read while the first
  // half's MFMAs run.  Between the two halves, each wave waits for its own loads of the next
  // stage, all waves meet at one barrier, the loads of the stage three ahead go out into
  // the buffer every wave has now finished reading, and the next stage's W chunks and first A
  // half are read while this stage's second-half MFMAs run.  The LDS reads of one stage thus
  // overlap the MFMAs of the one before, instead of all waves reading after a barrier while
  // the matrix cores wait.
  uint4 w16[4];
  bf16x8_t a0[MT], a1[MT];
  constexpr int MH = 0;
  // the W chunks and the first MH A fragments of the first half (read ahead, during the
  // previous stage's MFMAs); the other MH at the stage's start
  auto read_wa0 = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const unsigned char* Ab = lds + b * A_BYTES;
    const unsigned char* Wb = lds + DL_STAGES * A_BYTES + b * W_BYTES;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int r = 16 * (4 * wn + nt) + r16;
      w16[nt] = *reinterpret_cast<const uint4*>(Wb + r * 64 + 16 * (grp ^ ((r >> 2) & 3)));
    }
#pragma unroll
    for (int mt = 0; mt < MH; ++mt) {
      const int r = 16 * (MT * wm + mt) + r16;
      a0[mt] = *reinterpret_cast<const bf16x8_t*>(Ab + r * 128 + 16 * ((2 * grp) ^ ((r >> 1) & 7)));
    }
  };
  auto read_a0hi = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const unsigned char* Ab = lds + b * A_BYTES;
#pragma unroll
    for (int mt = MH; mt < MT; ++mt) {
      const int r = 16 * (MT * wm + mt) + r16;
      a0[mt] = *reinterpret_cast<const bf16x8_t*>(Ab + r * 128 + 16 * ((2 * grp) ^ ((r >> 1) & 7)));
    }
  };
  auto read_a1 = [&](auto bc) {
    constexpr int b = decltype(bc)::value;
    const unsigned char* Ab = lds + b * A_BYTES;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = 16 * (MT * wm + mt) + r16;
      a1[mt] = *reinterpret_cast<const bf16x8_t*>(Ab + r * 128 + 16 * ((2 * grp + 1) ^ ((r >> 1) & 7)));
    }
  };
  auto mfma_half = [&](const bf16x8_t (&af)[MT], const bf16x8_t (&bw)[4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bw[nt], acc[mt][nt], 0, 0, 0);
  };
  constexpr int LPS = 4 + WL;  // loads per wave and stage
  auto stage = [&](auto bc, int st) {
    constexpr int b = decltype(bc)::value;
    read_a0hi(bc);
    read_a1(bc);
    bf16x8_t bw[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bw[nt] = i8x8_to_bf16x8(make_uint2(w16[nt].x, w16[nt].y));
    mfma_half(a0, bw);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bw[nt] = i8x8_to_bf16x8(make_uint2(w16[nt].z, w16[nt].w));
    if (st + 1 < nsteps) {
      // this wave's loads of stage st + 1 have landed (only stage st + 2's remain) and its
      // reads of buffer b are done; after the barrier the same holds for every wave
      asm volatile("" ::: "memory");
      if (st + 2 < nsteps) __builtin_amdgcn_s_waitcnt(0x0070 | LPS);  // vmcnt <= LPS, lgkmcnt 0
      else __builtin_amdgcn_s_waitcnt(0x0070);                        // vmcnt 0, lgkmcnt 0
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (st + 3 < nsteps) issue(bc, st + 3);
      read_wa0(std::integral_constant<int, (b + 1) % DL_STAGES>{});
    }
    mfma_half(a1, bw);
  };
  issue(std::integral_constant<int, 0>{}, 0);
  if (nsteps > 1) issue(std::integral_constant<int, 1>{}, 1);
  if (nsteps > 2) issue(std::integral_constant<int, 2>{}, 2);
  // stage 0 landed for this wave (stages 1 and 2 may still be in flight), then for all
  asm volatile("" ::: "memory");
  if (nsteps > 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LPS));
  else if (nsteps > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | LPS);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_wa0(std::integral_constant<int, 0>{});
#pragma unroll 1
  for (int st = 0; st < nsteps; st += DL_STAGES) {
    stage(std::integral_constant<int, 0>{}, st);
    if (st + 1 < nsteps) stage(std::integral_constant<int, 1>{}, st + 1);
    if (st + 2 < nsteps) stage(std::integral_constant<int, 2>{}, st + 2);
  }

  if constexpr (EPI == EPI_STORE) {  // launched for q|k|v with the fused epilogue only
    {
      constexpr int TP = BN + 8;
      bf16_t* T = reinterpret_cast<bf16_t*>(lds);
      __syncthreads();  // every wave's last stage reads are done
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = n0 + wn * 64 + nt * 16 + r16;
        const float sc = a.scale[n < a.N ? n : 0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            T[(wm * 16 * MT + mt * 16 + 4 * grp + i) * TP + wn * 64 + nt * 16 + r16] = f2bf(acc[mt][nt][i] * sc);
      }
      __syncthreads();
      gemm_rope_tile<BM, BN, 512, 128>(a, T, m0, n0);  // (launched at head dim 128 only)
      return;
    }
  }
  if constexpr (EPI == EPI_SILU) {
    // gate/up: the tile's BN/2 outputs (columns n0/2 ..) go through LDS as bf16, then out as
    // whole 16-byte pieces of rows; the scales are requested once, before any store (a load
    // after stores waits for them, so per-column-block scale loads serialized the stores)
    constexpr int TP = BN / 2 + 8, PPR = BN / 16, NP = BM * PPR / 512;
    static_assert(BM * TP * 2 <= sizeof(lds) && BM * PPR % 512 == 0, "tile and passes");
    bf16_t* T = reinterpret_cast<bf16_t*>(lds);
    float sg[2], su[2];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int n = n0 + wn * 64 + pr * 32 + r16;  // gate row; its up row is n + GU_BLOCK
      sg[pr] = a.scale[n < a.N ? n : 0];
      su[pr] = a.scale[n + GU_BLOCK < a.N ? n + GU_BLOCK : 0];
    }
    __syncthreads();  // every wave's last stage reads are done
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = rbf(acc[mt][2 * pr][i] * sg[pr]);
          const float u = rbf(acc[mt][2 * pr + 1][i] * su[pr]);
          T[(wm * 16 * MT + mt * 16 + 4 * grp + i) * TP + wn * 32 + pr * 16 + r16] =
              f2bf(g / (1.0f + expf(-g)) * u);
        }
    __syncthreads();
    const int j0 = n0 / 2, nout = a.N / 2;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int idx = tid + 512 * u, row = idx / PPR, pc = idx % PPR;
      const int m = m0 + row, j = j0 + 8 * pc;
      if (m < a.M && j < nout)
        *reinterpret_cast<uint4*>(a.out + (size_t)m * a.ldo + j) =
            *reinterpret_cast<const uint4*>(&T[row * TP + 8 * pc]);
    }
    return;
  }
  if constexpr (EPI == EPI_RESID) {
    constexpr int TP = BN + 8;
    static_assert(BM * TP * 2 <= sizeof(lds), "the tile fits the stage buffers");
    bf16_t* T = reinterpret_cast<bf16_t*>(lds);
    __syncthreads();  // every wave's last stage reads are done
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = n0 + wn * 64 + nt * 16 + r16;
      const float sc = a.scale[n < a.N ? n : 0];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          T[(wm * 16 * MT + mt * 16 + 4 * grp + i) * TP + wn * 64 + nt * 16 + r16] = f2bf(acc[mt][nt][i] * sc);
    }
    __syncthreads();
    resid_tile_update<BM, BN, 512>(a, T, m0, n0);
    return;
  }
  // lane holds D[4*(lane/16)+i][lane%16] of each 16x16 tile: token rows, channel columns
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = n0 + wn * 64 + nt * 16 + r16;
    const float sc = a.scale[n < a.N ? n : 0];
    if (EPI == EPI_SILU) {
      if (nt & 1) continue;
      const int nu = n + GU_BLOCK;
      const float su = a.scale[nu < a.N ? nu : 0];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm * 16 * MT + mt * 16 + 4 * grp + i;
          if (m < a.M && nu < a.N) gemm_epilogue<EPI_SILU>(a, m, n, acc[mt][nt][i], acc[mt][nt + 1][i], sc, su);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm * 16 * MT + mt * 16 + 4 * grp + i;
          if (m < a.M && n < a.N) gemm_epilogue<EPI>(a, m, n, acc[mt][nt][i], 0.0f, sc, 0.0f);
        }
    }
  }
}

// Prefill GEMM for many token rows (the tile grid fills the GPU): a 128x128 output tile per
// work-group of 4 waves, each wave a 64x64 block of 4x4 MFMA 16x16x32 tiles, so every
// fragment read from LDS feeds four MFMAs (the 64x64-tile kernel's 32x32 wave blocks get
// two, which caps its MFMA rate at the LDS read bandwidth).  k advances 64 per LDS stage,
// double-buffered with one barrier per stage; the global loads of stage s+2 are in flight
// while stage s is multiplied, and the int8 weights become bf16 (exactly) when a stage is
// written to LDS.  Work-groups are dispatched round-robin over the 8 XCDs: XCD x takes a
// contiguous run of tiles in row-major (token-row, channel-column) order, so the tiles that
// share one L2 share token rows and walk neighbouring weight rows.  Residual inputs are read
// in the epilogue.  Two work-groups fit on a CU (68 KB of LDS each).
template <int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_big(QD_GEMM_PRELOAD_PARAMS, GemmArgs a) {
  QD_GEMM_PRELOAD_SET(a);
  constexpr int BM = 128, BN = 128, BK = 64;
  constexpr int OOB = (int)0x80000000;
  // LDS holds each 16-row x 32-k operand fragment in MFMA lane order: lane l's 8 values
  // (row l % 16, k 8*(l/16) ..) in 16-byte slot l ^ ((l / 16) % 4) of the fragment, so a
  // fragment read is 1 KB of consecutive bytes in which every 8 consecutive lanes hit 8
  // different bank groups; fragment f of a stage sits at 1088*f (odd fragments start 16
  // banks of 32 further along).  The staging writes of 8 consecutive lanes (one A row's 8
  // k chunks, or two W rows' 4 chunks) then also land on 8 different bank groups.
  constexpr int FRAG = 1088;                    // bytes per fragment slot
  constexpr int NFRAG = (BM / 16) * (BK / 32);  // 16 fragments per operand per stage
  __shared__ __align__(16) unsigned char Ab[2][NFRAG * FRAG];
  __shared__ __align__(16) unsigned char Wb[2][NFRAG * FRAG];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid & 1, wn = wid >> 1;
  const int grp = lane >> 4, r16 = lane & 15;
  const int ntn = (a.N + BN - 1) / BN, ntm = (a.M + BM - 1) / BM, ntiles = ntn * ntm;
  // XCD-contiguous tile order: XCD x = blockIdx % 8 owns tiles [start_x, start_x + count_x)
  const int q8 = ntiles >> 3, r8 = ntiles & 7, xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int t = xcd * q8 + min(xcd, r8) + loc;
  const int m0 = (t / ntn) * BM, n0 = (t % ntn) * BN;
  const int nsteps = (a.K + BK - 1) / BK;

  // rows past M (N) lie past the end of A (W) and read zero, as do k past K
  const __amdgpu_buffer_rsrc_t arsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, a.M * a.lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * a.K, 0x00020000);
  // staging, row-contiguous across lanes: A load j of thread tid is k chunk ca = tid % 8
  // (8 values) of tile row 32j + tid/8; W load j is k chunk cw = tid % 4 (16 codes, two
  // 8-value chunks once converted) of tile row 64j + tid/4
  const int ca = tid & 7, ra = tid >> 3, cw = tid & 3, rw = tid >> 2;
  auto slot = [](int row, int c) {  // byte offset of 8-value chunk c (of 8) of stage row row
    const int pos = (row & 15) + 16 * (c & 3);
    return ((row >> 4) * 2 + (c >> 2)) * FRAG + 16 * (pos ^ (c & 3));
  };
  struct Stage { uint4 a[4]; uint4 w[2]; };
  // (each offset passes through opaque_off: loads sharing one in-range condition were
  // otherwise turned into a branch per load, and the branch's wait drained every load in
  // flight)
  auto fetch = [&](int step, Stage& q) {
    const int ka = step * BK + 8 * ca, kw = step * BK + 16 * cw;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q.a[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             arsc, opaque_off(ka < a.K ? ((m0 + 32 * j + ra) * a.lda + ka) * 2 : OOB), 0, 0));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      q.w[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wrsc, opaque_off(kw < a.K ? (n0 + 64 * j + rw) * a.K + kw : OOB), 0, 0));
  };
  auto stash = [&](const Stage& q, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&Ab[buf][slot(32 * j + ra, ca)]) = q.a[j];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(64 * j + rw, 2 * cw)]) = i8x8_to_bf16x8(make_uint2(q.w[j].x, q.w[j].y));
      *reinterpret_cast<bf16x8_t*>(&Wb[buf][slot(64 * j + rw, 2 * cw + 1)]) = i8x8_to_bf16x8(make_uint2(q.w[j].z, q.w[j].w));
    }
  };
  const int rd = 16 * (lane ^ (grp & 3));  // this lane's slot in every fragment read

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Stage q[2];
  fetch(0, q[0]);
  fetch(1, q[1]);
  stash(q[0], 0);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int st = s0 + u;  // steps past the end multiply zeros (whole pairs of steps)
      fetch(st + 2, q[u]);    // into the slot step st vacated
      // (the next step's conversion stays behind this step's MFMAs, so its wait counts the
      // loads just issued)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        bf16x8_t af[4], bw[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *reinterpret_cast<const bf16x8_t*>(&Ab[u][((wm * 4 + mt) * 2 + sub) * FRAG + rd]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          bw[nt] = *reinterpret_cast<const bf16x8_t*>(&Wb[u][((wn * 4 + nt) * 2 + sub) * FRAG + rd]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bw[nt], acc[mt][nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      stash(q[u ^ 1], u ^ 1);  // step st + 1
      __syncthreads();
    }
  }

  // scales of this lane's four output channels (gate/up: two pairs), waited for once
  // here: the epilogue's stores count in the same counter as loads, so a wait for a scale
  // placed among the (conditional) stores would also wait for the stores before it
  float gsc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = n0 + wn * 64 + nt * 16 + r16;
    gsc[nt] = a.scale[n < a.N ? n : 0];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
  if constexpr (EPI == EPI_STORE) {
    if (a.fuse_rope) {
      gemm_big_rope_epilogue(a, reinterpret_cast<bf16_t*>(&Ab[0][0]), acc, gsc, m0, n0, wm, wn);
      return;
    }
  }
  if constexpr (EPI == EPI_RESID) {
    constexpr int TP = BN + 8;  // 128 x 136 bf16: exactly the A stage buffers
    static_assert(BM * TP * 2 <= sizeof(Ab), "the tile fits the A stage buffers");
    bf16_t* T = reinterpret_cast<bf16_t*>(&Ab[0][0]);
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          T[(wm * 64 + mt * 16 + 4 * grp + i) * TP + wn * 64 + nt * 16 + r16] = f2bf(acc[mt][nt][i] * gsc[nt]);
    __syncthreads();
    resid_tile_update<BM, BN, 256>(a, T, m0, n0);
    return;
  }
  // lane holds D[4*(lane/16)+i][lane%16] of each 16x16 tile: token rows, channel columns
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + mt * 16 + 4 * grp + i;
      if (m >= a.M) continue;
      if (EPI == EPI_SILU) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int ng = n0 + wn * 64 + pr * 32 + r16;
          if (ng + GU_BLOCK < a.N)
            gemm_epilogue<EPI_SILU>(a, m, ng, acc[mt][2 * pr][i], acc[mt][2 * pr + 1][i],
                                    gsc[2 * pr], gsc[2 * pr + 1]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int n = n0 + wn * 64 + nt * 16 + r16;
          if (n < a.N) gemm_epilogue<EPI>(a, m, n, acc[mt][nt][i], 0.0f, gsc[nt], 0.0f);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// batched decode GEMM on MFMA ("skinny": 2..64 token rows, weights swept once):
// Y[t][n] = scale[n] * sum_k X[t][k] * W[n][k], X bf16 (already RMS-normalized where the
// model normalizes), W int8 converted exactly to bf16 in registers.  The MFMA A operand is
// a 16-channel x 32-k slice of W, the B operand a 32-k x 16-token slice of X^T.  A
// work-group owns CTW 16-channel tiles; its four waves take interleaved 128-k blocks
// (each lane group streams 128 contiguous bytes of a weight row) and the partial sums
// meet in LDS.  The k order inside a block is permuted identically for both operands.
// operands of one 128-k block of a skinny tile: lane group grp covers k0 = kb + 32*grp
// .. +32 of the CTW weight rows and the TT token rows of this lane
template <int TT, int CTW>
struct SkinnyOps {
  uint4 w[CTW][2];
  uint4 x[TT][4];
};
// (lanes of padding token rows, past the batch, load nothing: their B operand is zero)
template <int TT, int CTW>
__device__ __forceinline__ void skinny_load(const int* const (&wrow)[CTW], const bool (&wok)[CTW],
                                            const bf16_t* const (&xrow)[TT], const bool (&xok)[TT],
                                            int K, int k0, SkinnyOps<TT, CTW>& o) {
  const bool kok = k0 < K;
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const uint4* src = reinterpret_cast<const uint4*>(wrow[c] + k0 / 4);
    o.w[c][0] = (kok && wok[c]) ? src[0] : make_uint4(0, 0, 0, 0);
    o.w[c][1] = (kok && wok[c]) ? src[1] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow[tt] + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) o.x[tt][q] = (kok && xok[tt]) ? src[q] : make_uint4(0, 0, 0, 0);
  }
}
template <int TT, int CTW>
__device__ __forceinline__ void skinny_mfma(const SkinnyOps<TT, CTW>& o, f32x4_t (&acc)[CTW][TT]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      const uint4 w16 = o.w[c][j >> 1];
      const uint2 w8 = (j & 1) ? make_uint2(w16.z, w16.w) : make_uint2(w16.x, w16.y);
      const bf16x8_t af = i8x8_to_bf16x8(w8);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        acc[c][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            af, __builtin_bit_cast(bf16x8_t, o.x[tt][j]), acc[c][tt], 0, 0, 0);
    }
  }
}
// blocks per load batch: every batch's loads are in flight before its first MFMA
template <int TT, int CTW>
constexpr int skinny_batch() { return TT * CTW >= 4 ? 2 : 3; }

// Row-contiguous activation loads (XS): load (tt, q) of a lane brings the 16 bytes of k
// chunk lane%16 (8 values) of the 128-k block for token 16tt + 4q + lane/16, so 16 lanes
// read one 256-byte row segment (the operand layout, 16 tokens per load, reads L2 several
// times slower).  The wave's own LDS slot then turns the chunks into the operand layout:
// token lane%16, k 32*(lane/16) + 8q.  Rows are XS_PITCH elements apart in the slot, so the
// 8 lanes of a fragment read hit 8 different bank groups.
constexpr int XS_PITCH = 136;
// The loads are buffer loads whose out-of-range offset reads zero: none sits in a branch,
// so the compiler's waits count exactly the loads each use needs.
template <int TT>
struct XRows {
  int off[TT][4];  // element offset in x of the lane's token row (clamped to a valid row)
  bool ok[TT][4];  // the token is in the batch
  int wb[2];       // byte offset in W of the lane's weight row of each 16-channel tile, or -1
  bf16_t* slot;    // this wave's LDS slot, TT*16 rows of XS_PITCH elements
  __amdgpu_buffer_rsrc_t xrs, wrs;  // x (unbounded: offsets are valid or out of range) and W
};
template <int TT>
__device__ __forceinline__ void xrows_init(const GemvArgs& a, bf16_t* slot, XRows<TT>& xr) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int tok = 16 * tt + 4 * q + grp;
      xr.ok[tt][q] = tok < a.nb;
      tok = tok < a.nb ? tok : a.nb - 1;
      xr.off[tt][q] = (a.x_rows ? a.x_rows[tok] : tok) * a.ldx;
    }
  xr.slot = slot;
  xr.wb[0] = xr.wb[1] = -1;
  xr.xrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, 0x7FFFFFFF, 0x00020000);
  xr.wrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * a.K, 0x00020000);
}
// the lane's weight rows of channel tile `tile` (CTW 16-channel tiles of it)
template <int TT, int CTW>
__device__ __forceinline__ void xrows_tile(const GemvArgs& a, int tile, XRows<TT>& xr) {
  const int r16 = threadIdx.x & 15;
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const int ch = tile * 16 * CTW + c * 16 + r16;
    xr.wb[c] = ch < a.N ? ch * a.K : -1;
  }
}
template <int TT, int CTW>
__device__ __forceinline__ void skinny_load_xs_x(const XRows<TT>& xr, int K, int kb, SkinnyOps<TT, CTW>& o) {
  constexpr int OOB = (int)0x80000000;
  const int kx = kb + 8 * (threadIdx.x & 15);
  const bool xk = kx < K;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o.x[tt][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xr.xrs, (xk && xr.ok[tt][q]) ? (xr.off[tt][q] + kx) * 2 : OOB, 0, 0));
}
template <int TT, int CTW>
__device__ __forceinline__ void skinny_load_xs_w(const XRows<TT>& xr, int K, int kb, SkinnyOps<TT, CTW>& o) {
  constexpr int OOB = (int)0x80000000;
  const int grp = (threadIdx.x & 63) >> 4;
  const int k0 = kb + 32 * grp;
  const bool kok = k0 < K;
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const int wo = (kok && xr.wb[c] >= 0) ? xr.wb[c] + k0 : OOB;
    o.w[c][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr.wrs, wo, 0, 0));
    o.w[c][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr.wrs, wo < 0 ? OOB : wo + 16, 0, 0));
  }
}
template <int TT, int CTW>
__device__ __forceinline__ void skinny_load_xs(const XRows<TT>& xr, int K, int kb, SkinnyOps<TT, CTW>& o) {
  skinny_load_xs_x<TT, CTW>(xr, K, kb, o);
  skinny_load_xs_w<TT, CTW>(xr, K, kb, o);
}
template <int TT, int CTW>
__device__ __forceinline__ void skinny_x_transpose(SkinnyOps<TT, CTW>& o, bf16_t* slot) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, r16 = lane & 15;
  // the wave's own slot: its LDS accesses run in program order; the fences keep the
  // compiler from moving them across each other
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(slot + (16 * tt + 4 * q + grp) * XS_PITCH + 8 * r16) = o.x[tt][q];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o.x[tt][q] = *reinterpret_cast<const uint4*>(slot + (16 * tt + r16) * XS_PITCH + 32 * grp + 8 * q);
}

// a wave's n blocks kb(i) = first + stride * ((i + rot) mod n), i < n, in load batches;
// XS: activations through the row-contiguous loads and the wave's LDS slot (xr)
template <int TT, int CTW, bool XS = false>
__device__ __forceinline__ void skinny_blocks(const int* const (&wrow)[CTW], const bool (&wok)[CTW],
                                              const bf16_t* const (&xrow)[TT],
                                              const bool (&xok)[TT], int K, int grp,
                                              int first, int stride, int n, int rot,
                                              f32x4_t (&acc)[CTW][TT], const bf16_t* x = nullptr,
                                              const XRows<TT>* xr = nullptr) {
  constexpr int U = skinny_batch<TT, CTW>();
  for (int ib = 0; ib < n; ib += U) {
    SkinnyOps<TT, CTW> ops[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int ii = ib + u + rot;
      ii = ii >= n ? ii - n : ii;
      const int kb = ib + u < n ? (first + stride * ii) * 128 : K;
      if constexpr (XS) skinny_load_xs<TT, CTW>(*xr, K, kb, ops[u]);
      else skinny_load<TT, CTW>(wrow, wok, xrow, xok, K, kb < K ? kb + 32 * grp : K, ops[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (XS) skinny_x_transpose<TT, CTW>(ops[u], xr->slot);
      skinny_mfma<TT, CTW>(ops[u], acc);
    }
  }
}

// stores one output element of a skinny tile: channel ch (tile-relative channel cr) of
// token tok from the raw dot products v (gate, up for SiLU), their scales and the residual
// (bf16 bits)
template <int EPI, int CTW>
__device__ __forceinline__ void skinny_out(const GemvArgs& a, int tile, int tok, int ch, int cr,
                                           const float (&v)[CTW], const float (&sc)[CTW], bf16_t res) {
  if (EPI == EPI_SILU) {
    if (tok < a.nb && ch + 16 < a.N) {
      const float g = rbf(v[0] * sc[0]), u = rbf(v[CTW - 1] * sc[CTW - 1]);
      a.out[(size_t)tok * a.ldo + tile * GU_BLOCK + cr] = f2bf(g / (1.0f + expf(-g)) * u);
    }
  } else if (tok < a.nb && ch < a.N) {
    const float y = v[0] * sc[0];
    bf16_t* o = a.out + (size_t)tok * a.ldo + ch;
    *o = (EPI == EPI_STORE) ? f2bf(y) : f2bf(bf2f(res) + rbf(y));
  }
}

template <int TT, int EPI, int NWS, bool XS = false>
__global__ __launch_bounds__(64 * NWS) void k_skinny(QD_SKINNY_PRELOAD_PARAMS, GemvArgs a) {
  QD_SKINNY_PRELOAD_SET(a);
  constexpr int CTW = (EPI == EPI_SILU) ? 2 : 1;
  constexpr int NACC = CTW * TT;
  __shared__ float red[NWS][NACC][4][64];
  __shared__ __align__(16) bf16_t xsl[XS ? NWS : 1][XS ? TT * 16 * XS_PITCH : 8];
  __shared__ unsigned long long kl[TT * 16][16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int grp = lane >> 4, r16 = lane & 15;
  const int ntiles = (a.N + 16 * CTW - 1) / (16 * CTW);
  unsigned long long best = 0ull;  // LOGITS: running best key of token tid (tid < 16*TT)

  // token rows of this lane's B operand, one per token tile
  const bf16_t* xrow[TT];
  bool xok[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int tok = tt * 16 + r16;
    xok[tt] = tok < a.nb;
    tok = tok < a.nb ? tok : a.nb - 1;
    const int xr = a.x_rows ? a.x_rows[tok] : tok;
    xrow[tt] = a.x + (size_t)xr * a.ldx;
  }
  XRows<TT> xr;
  if constexpr (XS) xrows_init<TT>(a, &xsl[wid][0], xr);

  // epilogue elements of this thread: e = tid + 64*NWS*q (token tile, row i, lane l)
  constexpr int NE = (TT * 256 + 64 * NWS - 1) / (64 * NWS);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    // their scales and residual inputs are requested before the k loop, so the epilogue
    // after the wave reduction does not wait for another round trip
    // (residuals as raw bits from a clamped index: no wait before the k loop's loads)
    float esc[NE][CTW];
    bf16_t eres[NE];
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int e = tid + 64 * NWS * q;
      const int tt = e / 256, i = (e / 64) % 4, l = e % 64;
      const int tok = tt * 16 + (l & 15);
      const int ch = tile * 16 * CTW + 4 * (l >> 4) + i;
      const bool ok = e < TT * 256 && tok < a.nb;
#pragma unroll
      for (int c = 0; c < CTW; ++c) {
        const bool sok = ok && ch + 16 * c < a.N;
        const float sv = a.scale[sok ? ch + 16 * c : 0];
        esc[q][c] = sok ? sv : 0.0f;
      }
      eres[q] = EPI == EPI_RESID ? a.out[(ok && ch < a.N) ? (size_t)tok * a.ldo + ch : 0] : (bf16_t)0;
    }
    f32x4_t acc[CTW][TT];
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[c][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int* wrow[CTW];
    bool wok[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      const int ch = tile * 16 * CTW + c * 16 + r16;
      wok[c] = ch < a.N;
      wrow[c] = reinterpret_cast<const int*>(a.W + (size_t)(wok[c] ? ch : 0) * K);
    }
    if constexpr (XS) xrows_tile<TT, CTW>(a, tile, xr);
    const int nkb = (K + 127) / 128;
    const int nmine = (nkb - wid + NWS - 1) / NWS;  // this wave's blocks: wid, wid+NWS, ...
    const int rot = nmine > 0 ? tile % nmine : 0;
    skinny_blocks<TT, CTW, XS>(wrow, wok, xrow, xok, K, grp, wid, NWS, nmine, rot, acc, a.x, &xr);
    // partial sums of the four waves meet in LDS
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wid][c * TT + tt][i][lane] = acc[c][tt][i];
    __syncthreads();
    // element (tt, i, l): channel tile*16*CTW + c*16 + 4*(l/16) + i, token tt*16 + l%16
#pragma unroll
    for (int q = 0; q < NE; ++q) {
      const int e = tid + 64 * NWS * q;
      if (e >= TT * 4 * 64) break;
      const int tt = e / 256, i = (e / 64) % 4, l = e % 64;  // e < TT*256
      const int tok = tt * 16 + (l & 15);
      float v[CTW];
#pragma unroll
      for (int c = 0; c < CTW; ++c) {
        v[c] = 0.0f;
#pragma unroll
        for (int w = 0; w < NWS; ++w) v[c] += red[w][c * TT + tt][i][l];
      }
      const int ch = tile * 16 * CTW + 4 * (l >> 4) + i;
      if (EPI == EPI_LOGITS) {
        unsigned long long k = 0ull;
        if (tok < a.nb && ch < a.N) {
          const float lv = v[0] * esc[q][0];
          if (a.logits) a.logits[(size_t)tok * a.ldl + ch] = lv;
          k = argmax_key(lv, ch);
        }
        kl[tok][4 * (l >> 4) + i] = k;
      } else {
        skinny_out<EPI, CTW>(a, tile, tok, ch, 4 * (l >> 4) + i, v, esc[q], eres[q]);
      }
    }
    if (EPI == EPI_LOGITS) {
      __syncthreads();
      if (tid < TT * 16) {
#pragma unroll
        for (int c = 0; c < 16; ++c) best = kl[tid][c] > best ? kl[tid][c] : best;
      }
    }
    __syncthreads();
  }
  if (EPI == EPI_LOGITS) lm_head_store(a, best, 64);
}

// RMSNorm folded in (batched decode, pre-norm activations, gain set): 8 waves, each holding
// all of its (at most NB) 128-k blocks in registers.  Every wave adds the squares of the raw
// activations it loaded per token; the partial sums meet in LDS and are added in wave order
// (fixed order), giving each token's 1/rms.  Each wave then normalizes its own registers,
// h = bf16(x * (1/rms) * g) with the gains staged in LDS, and runs the MFMAs as k_skinny does.
constexpr int SKN_WAVES = 8;
constexpr int SKN_MAX_K = 4096;  // 8 waves x 4 blocks x 128
// XS: activations loaded row-contiguously (16 lanes per 256-byte row segment, the layout
// that streams from L2 at full rate), squared and normalized in that layout, then turned
// into the matrix-core operand layout through the wave's own LDS slot before the MFMAs.
template <int TT, int EPI, int NB, bool XS = false>
__global__ __launch_bounds__(64 * SKN_WAVES) void k_skinny_norm(QD_SKINNY_PRELOAD_PARAMS, GemvArgs a) {
  QD_SKINNY_PRELOAD_SET(a);
  constexpr int NWS = SKN_WAVES;
  constexpr int CTW = (EPI == EPI_SILU) ? 2 : 1;
  constexpr int NACC = CTW * TT;
  constexpr int NE = (TT * 256 + 64 * NWS - 1) / (64 * NWS);
  __shared__ float red[NWS][NACC][4][64];
  __shared__ __align__(16) float gs[SKN_MAX_K];
  __shared__ float sq[NWS][TT * 16];
  __shared__ float rinv[TT * 16];
  __shared__ __align__(16) bf16_t xsl[XS ? NWS : 1][XS ? TT * 16 * XS_PITCH : 8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int grp = lane >> 4, r16 = lane & 15;
  const int tile = blockIdx.x;

  const bf16_t* xrow[TT];
  bool xok[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int tok = tt * 16 + r16;
    xok[tt] = tok < a.nb;
    tok = tok < a.nb ? tok : a.nb - 1;
    const int xr = a.x_rows ? a.x_rows[tok] : tok;
    xrow[tt] = a.x + (size_t)xr * a.ldx;
  }
  const int* wrow[CTW];
  bool wok[CTW];
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const int ch = tile * 16 * CTW + c * 16 + r16;
    wok[c] = ch < a.N;
    wrow[c] = reinterpret_cast<const int*>(a.W + (size_t)(wok[c] ? ch : 0) * K);
  }
  XRows<TT> xr;
  if constexpr (XS) {
    xrows_init<TT>(a, &xsl[wid][0], xr);
    xrows_tile<TT, CTW>(a, tile, xr);
  }
  // all of this wave's blocks (wid, wid + 8, ...) in one batch.  XS: every load of a lane
  // covers k = 128*kb + 8*r16 .. +8, so the lane's 8 gains of each block are requested
  // with its activations, before the weights: the RMSNorm then waits for neither the
  // weights nor an LDS staging of the gains (which would wait for every load in flight)
  SkinnyOps<TT, CTW> ops[NB];
  float4 gx[XS ? NB : 1][2];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int kb = wid + NWS * u;
    if constexpr (XS) {
      const int kx = kb * 128 + 8 * r16;
      const float4* g4 = reinterpret_cast<const float4*>(a.gain + (kx < K ? kx : 0));
      gx[u][0] = g4[0];
      gx[u][1] = g4[1];
      skinny_load_xs_x<TT, CTW>(xr, K, kb * 128 < K ? kb * 128 : K, ops[u]);
    } else {
      skinny_load<TT, CTW>(wrow, wok, xrow, xok, K, kb * 128 < K ? kb * 128 + 32 * grp : K, ops[u]);
    }
  }
  if constexpr (XS) {  // every block's weights after every block's activations (loads retire
                       // in order: the squares would otherwise wait for weights)
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kb = wid + NWS * u;
      skinny_load_xs_w<TT, CTW>(xr, K, kb * 128 < K ? kb * 128 : K, ops[u]);
    }
  }
  // epilogue inputs (residuals as raw bits from a clamped index)
  float esc[NE][CTW];
  bf16_t eres[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 64 * NWS * q;
    const int tt = e / 256, i = (e / 64) % 4, l = e % 64;
    const int tok = tt * 16 + (l & 15);
    const int ch = tile * 16 * CTW + 4 * (l >> 4) + i;
    const bool ok = e < TT * 256 && tok < a.nb;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      const bool sok = ok && ch + 16 * c < a.N;
      const float sv = a.scale[sok ? ch + 16 * c : 0];
      esc[q][c] = sok ? sv : 0.0f;
    }
    eres[q] = EPI == EPI_RESID ? a.out[(ok && ch < a.N) ? (size_t)tok * a.ldo + ch : 0] : (bf16_t)0;
  }
  // the gains, staged once per work-group (the LDS store waits for every load above)
  if constexpr (!XS)
    for (int k = tid * 4; k < K; k += 64 * NWS * 4)
      *reinterpret_cast<float4*>(&gs[k]) = *reinterpret_cast<const float4*>(a.gain + k);
  if constexpr (XS) {
    // load (tt, q) of a lane holds 8 values of token 16tt + 4q + grp: squares per load,
    // then over the 16 lanes of the group
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s2 = 0.0f;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const uint4 v = ops[u].x[tt][q];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xFFFF0000u);
            s2 += lo * lo + hi * hi;
          }
        }
        s2 = row16_sum(s2);
        if (r16 == 0) sq[wid][tt * 16 + 4 * q + grp] = s2;
      }
  } else {
    // squares of this lane's raw activations per token row, then over the four lane groups
    float ss[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      ss[tt] = 0.0f;
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = ops[u].x[tt][q];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xFFFF0000u);
            ss[tt] += lo * lo + hi * hi;
          }
        }
      ss[tt] = xor32_sum(xor16_sum(ss[tt]));
      if (grp == 0) sq[wid][tt * 16 + r16] = ss[tt];
    }
  }
  __syncthreads();
  if (tid < TT * 16) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NWS; ++w) t += sq[w][tid];
    rinv[tid] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
  // (XS: 1/rms of token 16tt + 4q + grp; else of token 16tt + r16)
  float inv[TT][XS ? 4 : 1];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < (XS ? 4 : 1); ++q) inv[tt][q] = rinv[XS ? tt * 16 + 4 * q + grp : tt * 16 + r16];

  f32x4_t acc[CTW][TT];
#pragma unroll
  for (int c = 0; c < CTW; ++c)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[c][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int kb = (wid + NWS * u) * 128;
    if (kb >= K) break;  // wave-uniform; no load is issued after this point
    // XS: every load of the lane covers k = kb + 8*r16 .. +8; else load q covers
    // kb + 32*grp + 8q .. +8
    const int k0 = XS ? kb + 8 * r16 : kb + 32 * grp;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // gains (XS: from registers, else from LDS); positions past K hold zero activations
      const int kq = XS ? k0 : k0 + 8 * q;
      const int kg = kq < K ? kq : 0;
      const float4 g0 = XS ? gx[XS ? u : 0][0] : *reinterpret_cast<const float4*>(&gs[kg]);
      const float4 g1 = XS ? gx[XS ? u : 0][1] : *reinterpret_cast<const float4*>(&gs[kg + 4]);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const float iv = inv[tt][XS ? q : 0];
        const uint4 v = ops[u].x[tt][q];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        uint32_t o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(w4[e] << 16) * iv * gv[2 * e];
          const float hi = __uint_as_float(w4[e] & 0xFFFF0000u) * iv * gv[2 * e + 1];
          o4[e] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
        }
        ops[u].x[tt][q] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
      }
    }
    if constexpr (XS) skinny_x_transpose<TT, CTW>(ops[u], xr.slot);
    skinny_mfma<TT, CTW>(ops[u], acc);
  }
#pragma unroll
  for (int c = 0; c < CTW; ++c)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wid][c * TT + tt][i][lane] = acc[c][tt][i];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 64 * NWS * q;
    if (e >= TT * 4 * 64) break;
    const int tt = e / 256, i = (e / 64) % 4, l = e % 64;
    const int tok = tt * 16 + (l & 15);
    float v[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      v[c] = 0.0f;
#pragma unroll
      for (int w = 0; w < NWS; ++w) v[c] += red[w][c * TT + tt][i][l];
    }
    const int ch = tile * 16 * CTW + 4 * (l >> 4) + i;
    skinny_out<EPI, CTW>(a, tile, tok, ch, 4 * (l >> 4) + i, v, esc[q], eres[q]);
  }
}

// Split-K form for projections with few channel tiles: work-group blockIdx = tile * S + s
// sums the 128-k blocks [s*nkb/S, (s+1)*nkb/S) of one tile, one block per wave per pass.
// Each work-group's tile partial goes out with agent-coherent stores; the work-group that
// counts in last adds the S partials in split order (fixed order: the result does not
// depend on arrival order) and runs the epilogue.  No work-group waits for another.
template <int TT, int EPI, int NWS, bool XS = false>
__global__ __launch_bounds__(64 * NWS) void k_skinny_split(QD_SKINNY_PRELOAD_PARAMS, GemvArgs a) {
  QD_SKINNY_PRELOAD_SET(a);
  constexpr int CTW = (EPI == EPI_SILU) ? 2 : 1;
  constexpr int NACC = CTW * TT;
  constexpr int NE = (TT * 256 + 64 * NWS - 1) / (64 * NWS);
  __shared__ float red[NWS][NACC][4][64];
  __shared__ __align__(16) bf16_t xsl[XS ? NWS : 1][XS ? TT * 16 * XS_PITCH : 8];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K, S = a.ksplit;
  const int grp = lane >> 4, r16 = lane & 15;
  const int tile = blockIdx.x / S, s = blockIdx.x - tile * S;

  const bf16_t* xrow[TT];
  bool xok[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int tok = tt * 16 + r16;
    xok[tt] = tok < a.nb;
    tok = tok < a.nb ? tok : a.nb - 1;
    const int xr = a.x_rows ? a.x_rows[tok] : tok;
    xrow[tt] = a.x + (size_t)xr * a.ldx;
  }
  XRows<TT> xr;
  if constexpr (XS) {
    xrows_init<TT>(a, &xsl[wid][0], xr);
    xrows_tile<TT, CTW>(a, tile, xr);
  }
  const int* wrow[CTW];
  bool wok[CTW];
#pragma unroll
  for (int c = 0; c < CTW; ++c) {
    const int ch = tile * 16 * CTW + c * 16 + r16;
    wok[c] = ch < a.N;
    wrow[c] = reinterpret_cast<const int*>(a.W + (size_t)(wok[c] ? ch : 0) * K);
  }
  f32x4_t acc[CTW][TT];
#pragma unroll
  for (int c = 0; c < CTW; ++c)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[c][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nkb = (K + 127) / 128;
  const int b0 = s * nkb / S, b1 = (s + 1) * nkb / S;
  const int nmine = (b1 - b0 - wid + NWS - 1) / NWS;
  skinny_blocks<TT, CTW, XS>(wrow, wok, xrow, xok, K, grp, b0 + wid, NWS, nmine > 0 ? nmine : 0, 0, acc,
                             a.x, &xr);

  // epilogue inputs, requested while the partials are exchanged
  float esc[NE][CTW];
  bf16_t eres[NE];
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 64 * NWS * q;
    const int tt = e / 256, i = (e / 64) % 4, l = e % 64;
    const int tok = tt * 16 + (l & 15);
    const int ch = tile * 16 * CTW + 4 * (l >> 4) + i;
    const bool ok = e < TT * 256 && tok < a.nb;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      const bool sok = ok && ch + 16 * c < a.N;
      const float sv = a.scale[sok ? ch + 16 * c : 0];
      esc[q][c] = sok ? sv : 0.0f;
    }
    eres[q] = EPI == EPI_RESID ? a.out[(ok && ch < a.N) ? (size_t)tok * a.ldo + ch : 0] : (bf16_t)0;
  }

#pragma unroll
  for (int c = 0; c < CTW; ++c)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wid][c * TT + tt][i][lane] = acc[c][tt][i];
  __syncthreads();
  // this work-group's partial: element e of accumulator c at part[((tile*S + s)*CTW + c)*TT*256 + e]
  float v[NE][CTW];
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 64 * NWS * q;
    const int tt = e / 256, i = (e / 64) % 4, l = e % 64;
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      v[q][c] = 0.0f;
      if (e < TT * 256) {
#pragma unroll
        for (int w = 0; w < NWS; ++w) v[q][c] += red[w][c * TT + tt][i][l];
        __hip_atomic_store(a.kpart + ((size_t)blockIdx.x * CTW + c) * (TT * 256) + e, v[q][c],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // every store of this work-group has completed before thread 0 counts it in
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned t = __hip_atomic_fetch_add(a.kcnt + tile, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    is_last = t == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!is_last) return;

  // the S partials of the tile, eight splits per round trip (agent-coherent buffer loads;
  // an offset past the buffer's end reads zero and is not added)
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kpart + (size_t)tile * S * CTW * TT * 256), 0, S * CTW * TT * 256 * 4, 0x00020000);
#pragma unroll
  for (int q = 0; q < NE; ++q) {
    const int e = tid + 64 * NWS * q;
    if (e >= TT * 256) break;
    const int tt = e / 256, i = (e / 64) % 4, l = e % 64;
    const int tok = tt * 16 + (l & 15);
    const int ch = tile * 16 * CTW + 4 * (l >> 4) + i;
    float tot[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) tot[c] = 0.0f;
    for (int s0 = 0; s0 < S; s0 += 8) {
      float pv[8][CTW];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
          const int sj = s0 + j;
          const int off = (sj < S && sj != s) ? ((sj * CTW + c) * (TT * 256) + e) * 4 : (int)0x80000000;
          pv[j][c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, 16));
        }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
          const int sj = s0 + j;
          if (sj < S) tot[c] += sj == s ? v[q][c] : pv[j][c];
        }
    }
    skinny_out<EPI, CTW>(a, tile, tok, ch, 4 * (l >> 4) + i, tot, esc[q], eres[q]);
  }
  if (tid == 0) __hip_atomic_store(a.kcnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Batched LM head (vocabulary-sized N): a work-group owns 4 waves x LMT 16-channel tiles
// and walks K in chunks; each chunk of the activations is staged once in LDS for all
// 4*LMT tiles (the activations are read from L2 once per work-group instead of once per
// tile), and every tile's accumulators stay in registers across the chunks.  K advances
// 128 per step; the weights of step s + 1 are requested (branch-free buffer loads, tiles
// past the vocabulary read zero) before step s is multiplied, so a wave always has the
// next step's rows in flight instead of waiting out one memory round trip per step.
// NS > 0: K = 128 NS, the step loop fully unrolled (a loop back edge with loads in flight
// would make the compiler wait for them to move registers)
constexpr int LMT = 4;
template <int TT, int NS>
__global__ __launch_bounds__(256) void k_lm_skinny(QD_SKINNY_PRELOAD_PARAMS, GemvArgs a) {
  QD_SKINNY_PRELOAD_SET(a);
  constexpr int KC = 1024 / TT;                 // k per chunk: LDS = 16*TT rows x KC
  constexpr int OOB = (int)0x80000000;
  __shared__ __align__(16) bf16_t xs[TT * 16][KC + 8];
  __shared__ unsigned long long wkey[4][TT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int grp = lane >> 4, r16 = lane & 15;
  const int ntiles = (a.N + 15) / 16;
  f32x4_t acc[LMT][TT];
#pragma unroll
  for (int t = 0; t < LMT; ++t)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[t][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int tile[LMT], wofs[LMT];  // this lane's weight row offset, or -1 past the vocabulary
#pragma unroll
  for (int t = 0; t < LMT; ++t) {
    tile[t] = (blockIdx.x * LMT + t) * 4 + wid;
    const int ch = tile[t] * 16 + r16;
    wofs[t] = (tile[t] < ntiles && ch < a.N) ? ch * K : -1;
  }
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.W, 0, a.N * K, 0x00020000);
  const int nsteps = NS > 0 ? NS : (K + 127) / 128;
  // step s: k = 128 s + 32 grp .. + 31 of each of the lane's rows
  auto wload = [&](int st, uint4 (&wv)[LMT][2]) {
    const int k = st * 128 + 32 * grp;
#pragma unroll
    for (int t = 0; t < LMT; ++t) {
      const bool ok = wofs[t] >= 0 && k < K && st < nsteps;
      wv[t][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, ok ? wofs[t] + k : OOB, 0, 0));
      wv[t][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, ok ? wofs[t] + k + 16 : OOB, 0, 0));
    }
  };
  // activation staging: a chunk is TT*16 rows x KC/8 16-byte pieces, NST per thread
  // (piece idx = tid + 256 u: row idx / (KC/8), piece idx % (KC/8)); the source rows are
  // looked up once, and a chunk's pieces are requested together (buffer loads; rows past
  // the batch and k past K read zero)
  constexpr int VPR = KC / 8, NST = TT * 16 * VPR / 256;
  static_assert(TT * 16 * VPR % 256 == 0, "whole staging passes");
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, 0x7FFFFFFF, 0x00020000);
  int xoff[NST];
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int r = (tid + 256 * u) / VPR, c = (tid + 256 * u) % VPR;
    const int rc = r < a.nb ? r : 0;
    const int xr = a.x_rows ? a.x_rows[rc] : rc;
    xoff[u] = r < a.nb ? (xr * a.ldx + 8 * c) * 2 : -1;
  }
  uint4 wa[LMT][2], wb[LMT][2];
  wload(0, wa);
  // the scales of this lane's output channels are requested before the k loop
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)a.scale, 0, a.N * 4, 0x00020000);
  float lsc[LMT][4];
#pragma unroll
  for (int t = 0; t < LMT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tile[t] * 16 + 4 * grp + i;
      lsc[t][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                srs, (tile[t] < ntiles && ch < a.N) ? ch * 4 : OOB, 0, 0));
    }
  auto step = [&](int st, const uint4 (&wv)[LMT][2], uint4 (&wn)[LMT][2]) {
    const int kc = (st * 128) / KC * KC;  // this step's chunk
    if (st * 128 == kc) {
      uint4 v[NST];
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int c = (tid + 256 * u) % VPR;
        const bool ok = xoff[u] >= 0 && kc + 8 * c < K;
        v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, ok ? xoff[u] + kc * 2 : OOB, 0, 0));
      }
      __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int r = (tid + 256 * u) / VPR, c = (tid + 256 * u) % VPR;
        *reinterpret_cast<uint4*>(&xs[r][8 * c]) = v[u];
      }
      __syncthreads();
    }
    wload(st + 1, wn);  // the next step's rows go out before this step's products
    const int k0 = st * 128 - kc + 32 * grp;  // within the chunk
    const bool kok = st * 128 + 32 * grp < K;
    uint4 xv[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[tt][q] = kok ? *reinterpret_cast<const uint4*>(&xs[tt * 16 + r16][k0 + 8 * q]) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < LMT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 w16 = wv[t][j >> 1];
        const uint2 w8 = (j & 1) ? make_uint2(w16.z, w16.w) : make_uint2(w16.x, w16.y);
        const bf16x8_t af = i8x8_to_bf16x8(w8);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_t, xv[tt][j]),
                                                              acc[t][tt], 0, 0, 0);
      }
    }
  };
  if constexpr (NS > 0) {
#pragma unroll
    for (int st = 0; st < NS; st += 2) {
      step(st, wa, wb);
      if (st + 1 < NS) step(st + 1, wb, wa);
    }
  } else {
    for (int st = 0; st < nsteps; st += 2) {
      step(st, wa, wb);
      if (st + 1 < nsteps) step(st + 1, wb, wa);
    }
  }
  // lane holds channel tile*16 + 4*grp + i, token tt*16 + r16
  unsigned long long best[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    best[tt] = 0ull;
    const int tok = tt * 16 + r16;
#pragma unroll
    for (int t = 0; t < LMT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = tile[t] * 16 + 4 * grp + i;
        if (tok < a.nb && tile[t] < ntiles && ch < a.N) {
          const float lv = acc[t][tt][i] * lsc[t][i];
          if (a.logits) a.logits[(size_t)tok * a.ldl + ch] = lv;
          const unsigned long long k = argmax_key(lv, ch);
          best[tt] = k > best[tt] ? k : best[tt];
        }
      }
    }
    unsigned long long t1 = shfl_xor_u64(best[tt], 16);
    best[tt] = t1 > best[tt] ? t1 : best[tt];
    t1 = shfl_xor_u64(best[tt], 32);
    best[tt] = t1 > best[tt] ? t1 : best[tt];
    if (lane < 16) wkey[wid][tt * 16 + lane] = best[tt];
  }
  __syncthreads();
  unsigned long long mine = 0ull;
  if (tid < TT * 16) {
    mine = wkey[0][tid];
    for (int w = 1; w < 4; ++w) mine = wkey[w][tid] > mine ? wkey[w][tid] : mine;
  }
  lm_head_store(a, mine, TT * 16);
}

// ------------------------------------------------------------------------------------------
// QK-norm + RoPE + KV-cache write.  Work-group (row, head group): each wave owns one head
// slot of the row (q heads, then k heads, then v heads), so a wave makes one round trip.
// q and k heads: RMSNorm over head_dim with a shared gain, then rotate-half RoPE at
// the row's position; q is written back in place, k and v go to the cache.
__global__ __launch_bounds__(256) void k_qk_rope(QD_ROPE_PRELOAD_PARAMS, RopeArgs a) {
  QD_ROPE_PRELOAD_SET(a);
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int hh = blockIdx.y * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);
  if (hh >= a.H + 2 * a.KV) return;  // whole waves; the kernel has no block barrier
  const int D = a.D, half = D / 2;
  const int slot = a.row_slot[r], p = a.row_pos[r];
  bf16_t* src = a.qkv + (size_t)r * a.ldqkv + (size_t)hh * D;
  if (hh >= a.H + a.KV) {
    const int g = hh - a.H - a.KV;
    bf16_t* dst = a.vcache + (((size_t)slot * a.KV + g) * a.max_ctx + p) * D;
    for (int i = lane; i < D; i += 64) dst[i] = src[i];
    return;
  }
  const bool isq = hh < a.H;
  const float* gn = isq ? a.q_gain : a.k_gain;
  const float2* tab = a.rope + (size_t)p * half;
  // every input of the head requested at once, from clamped (valid) indices
  bf16_t xb1[2], xb2[2];
  float g1[2], g2[2];
  float2 cs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    const int ic = i < half ? i : 0;
    xb1[j] = src[ic];
    xb2[j] = src[ic + half];
    g1[j] = gn[ic];
    g2[j] = gn[ic + half];
    cs[j] = tab[ic];
  }
  float x1[2], x2[2], ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool ok = lane + 64 * j < half;
    x1[j] = ok ? bf2f(xb1[j]) : 0.0f;
    x2[j] = ok ? bf2f(xb2[j]) : 0.0f;
    ss += x1[j] * x1[j] + x2[j] * x2[j];
  }
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)D + a.eps);
  bf16_t* dst = src;
  if (!isq) {
    const int g = hh - a.H;
    dst = a.kcache + (((size_t)slot * a.KV + g) * a.max_ctx + p) * D;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    if (i < half) {
      const float y1 = rbf(x1[j] * rinv * g1[j]);
      const float y2 = rbf(x2[j] * rinv * g2[j]);
      dst[i] = f2bf(y1 * cs[j].x - y2 * cs[j].y);
      dst[i + half] = f2bf(y2 * cs[j].x + y1 * cs[j].y);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Decode attention for one token row b, one KV head g and one split of positions.
// Fused in front: RMSNorm (shared [D] gain) and rotate-half RoPE at position p of the
// group's G query heads and of its key head, done in LDS from the raw projections; the
// split that holds position p writes the new K and V rows to the cache and every split
// uses the fresh rows for p from LDS.  Each wave owns 16 positions of every 64-position
// chunk and keeps its own online-softmax state in base 2 (no block barrier inside the
// loop); K and V tiles, all 16-byte loads, are requested one chunk ahead, the first ones
// before the prologue.  A lane's scores become the P*V lanes' probabilities through a
// per-wave LDS slot, and each P*V lane accumulates 8 output dims of its own positions
// across all chunks (reduced across lanes once at the end).  The waves merge in LDS at the
// end.  Fused behind: with several splits, each writes its partial (base-2 max, sum,
// unnormalized output); the split that finishes last merges them.
// WIDE: more than SB = 8 splits, merged by the batched path below (its own instantiation, so
// the short-context kernel keeps its registers and LDS)
// The fields of the first dependent loads (the row's slot, its position, the K/V tile and
// projection addresses) come as leading scalar arguments, preloaded into SGPRs at wave launch.
template <int D, int G, int NW, bool WIDE>
__global__ __launch_bounds__(64 * NW) void k_attn_dec(const int* row_slot_, const int* pos_,
                                                      const bf16_t* qkv_, bf16_t* kcache_, bf16_t* vcache_,
                                                      int ldqkv_, int KV_, int max_ctx_, int split_len_,
                                                      AttnDecArgs a) {
  a.row_slot = row_slot_;
  a.pos = pos_;
  a.qkv = qkv_;
  a.kcache = kcache_;
  a.vcache = vcache_;
  a.ldqkv = ldqkv_;
  a.KV = KV_;
  a.max_ctx = max_ctx_;
  a.split_len = split_len_;
  constexpr int NT = 64 * NW;              // threads
  constexpr int CHW = 16 * NW;             // positions per iteration
  constexpr int HALF = D / 2;
  // scores: 4 lanes per position, lane part of position tl holds key dims 32j + 8*part .. +8
  // (16-byte chunks j < KV4), so the 4 lanes of a position read 64 contiguous bytes per load
  constexpr int KV4 = D / 32;
  // P*V: lane (vch = lane % CL, vu = lane / CL) holds dims 8*vch .. +8 of the wave's
  // positions vu, vu + PSL, ... (VR rows as 16-byte loads; CL lanes cover a 256-byte row)
  // and accumulates its own partial output over every chunk; the PSL position slots are
  // added once, after the last chunk
  constexpr int CL = D / 8, PSL = 64 / CL, VR = 16 / PSL;
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ __align__(16) float qs[G][D];
  __shared__ __align__(16) bf16_t qb[G][D];  // the same q as bf16 (it is bf16-exact)
  __shared__ float kn[D], vn[D];
  __shared__ float wm[NW][G], wl[NW][G];
  __shared__ float wo[NW][G][D];
  __shared__ __align__(16) float ps[NW][G][16];  // each wave's probabilities of its 16 positions
  __shared__ int last_flag;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // wave index as a scalar: per-wave choices (which head, which gain vector) stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tl = lane >> 2, part = lane & 3;
  const int sl = a.row_slot ? a.row_slot[b] : b;  // KV slot of this row
  const int p = a.pos[sl];
  const int n = p + 1;
  const int t_begin = s * a.split_len;
  const int t_end = min(n, t_begin + a.split_len);
  const bf16_t* row = a.qkv + (size_t)b * a.ldqkv;
  const float2* tab = a.rope + (size_t)p * HALF;
  bf16_t* Kb = a.kcache + ((size_t)sl * a.KV + g) * a.max_ctx * D;
  bf16_t* Vb = a.vcache + ((size_t)sl * a.KV + g) * a.max_ctx * D;
  const bool owner = (t_begin <= p) && (p < t_begin + a.split_len);
  const int vch = lane % CL, vu = lane / CL;

  // ---- K/V tiles of the first chunk, requested before anything else ----
  // Buffer loads: a position outside the split (or p itself, taken from LDS) reads zero
  // through an out-of-range offset, so no load sits in a branch and every wait counts
  // exactly the loads it needs.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(Kb, 0, a.max_ctx * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(Vb, 0, a.max_ctx * D * 2, 0x00020000);
  constexpr int OOB = (int)0x80000000;
  uint4 kc[KV4], kx[KV4];
  uint4 vc[VR], vx[VR];
  // (the wave index here is the per-lane one: with scalar validity conditions the
  // compiler branches around groups of loads instead of selecting offsets)
  const int wv = tid >> 6;
  auto load_tiles = [&](uint4 (&kk)[KV4], uint4 (&vv)[VR], int t0) {
    const int t = t0 + 16 * wv + tl;
    const bool kok = t < t_end && t != p;
#pragma unroll
    for (int j = 0; j < KV4; ++j)
      kk[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            krs, kok ? (t * D + 32 * j + 8 * part) * 2 : OOB, 0, 0));
#pragma unroll
    for (int i = 0; i < VR; ++i) {
      const int tv = t0 + 16 * wv + vu + PSL * i;
      const bool ok = tv < t_end && tv != p;
      vv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            vrs, ok ? (tv * D + 8 * vch) * 2 : OOB, 0, 0));
    }
  };
  // ---- QK-norm + RoPE of the G query heads and the key head; copy of v ----
  // The projections, gains and RoPE factors of this wave's first head are requested before
  // the K/V tiles: a wave's loads retire in order, so the prologue then waits only for its
  // own inputs while the tiles are still in flight.
  auto head_src = [&](int hh) {
    return hh < G ? row + (size_t)(g * G + hh) * D : row + (size_t)(a.H + g) * D;
  };
  // Loads from clamped (always valid) indices, projections kept as raw bits until used: a
  // load in a branch, or converted where it lands, makes the wave wait for it there.
  constexpr int HJ = HALF > 64 ? 2 : 1;  // 64-lane passes over half a head
  bf16_t xb1[HJ], xb2[HJ];
  float gg1[HJ], gg2[HJ];
  float2 cs2[HJ];
  auto head_load = [&](int hh) {
    const bf16_t* src = head_src(hh);
    const float* gn = hh < G ? a.q_gain : a.k_gain;
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const int i = lane + 64 * j;
      const int ic = i < HALF ? i : 0;
      xb1[j] = src[ic];
      xb2[j] = src[ic + HALF];
      gg1[j] = gn[ic];
      gg2[j] = gn[ic + HALF];
      cs2[j] = tab[ic];
    }
  };
  const bf16_t* vsrc = row + (size_t)(a.H + a.KV + g) * D;
  const int vi = tid < D ? tid : 0;
  const bf16_t vfirst = vsrc[vi];
  // waves past the G + 1 heads redo the key head and drop the result: the first head is
  // processed by every wave in straight-line code, so its loads stay ahead of the tiles
  // (behind a branch the compiler would sink them below the tile loads and then wait for
  // every tile before the first head)
  const int hh0 = wid <= G ? wid : G;
  head_load(hh0);
  load_tiles(kc, vc, t_begin);  // unconditional: an empty split reads zeros
  auto head_norm_rope = [&](int hh, bool live) {
    const bool isq = hh < G;
    float ss = 0.0f, x1[HJ], x2[HJ];
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const bool ok = lane + 64 * j < HALF;
      x1[j] = ok ? bf2f(xb1[j]) : 0.0f;
      x2[j] = ok ? bf2f(xb2[j]) : 0.0f;
      ss += x1[j] * x1[j] + x2[j] * x2[j];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const int i = lane + 64 * j;
      // every wave stores its head to LDS (the waves past the G + 1 heads write the same key
      // values as the key head's wave), so nothing here is conditional on the wave and no
      // input load is sunk into a branch; the cache row is written once
      const float y1 = rbf(x1[j] * inv * gg1[j]);
      const float y2 = rbf(x2[j] * inv * gg2[j]);
      const float2 cs = cs2[j];
      const bf16_t o1 = f2bf(y1 * cs.x - y2 * cs.y), o2 = f2bf(y2 * cs.x + y1 * cs.y);
      if (i < HALF) {
        if (isq) {
          qs[hh][i] = bf2f(o1);
          qs[hh][i + HALF] = bf2f(o2);
          qb[hh][i] = o1;
          qb[hh][i + HALF] = o2;
        } else {
          kn[i] = bf2f(o1);
          kn[i + HALF] = bf2f(o2);
          if (owner && live) {
            Kb[(size_t)p * D + i] = o1;
            Kb[(size_t)p * D + i + HALF] = o2;
          }
        }
      }
    }
  };
  head_norm_rope(hh0, wid <= G);
  for (int hh = wid + NW; hh <= G; hh += NW) {
    head_load(hh);
    head_norm_rope(hh, true);
  }
  for (int i = tid; i < D; i += NT) {
    const bf16_t v = i == tid ? vfirst : vsrc[i];
    vn[i] = bf2f(v);
    if (owner) Vb[(size_t)p * D + i] = v;
  }
  __syncthreads();

  // scores in base 2: z = q.k * log2(e) / sqrt(D), weights 2^(z - m)
  const float scale2 = LOG2E / sqrtf((float)D);
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
  }
  for (int t0 = t_begin; t0 < t_end; t0 += CHW) {
    const int t = t0 + 16 * wid + tl;
    // scores of this lane's position (4 lanes per position, D/4 key elements each)
    float sp[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sp[h] = 0.0f;
    if (t == p) {
#pragma unroll
      for (int j = 0; j < KV4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dd = 32 * j + 8 * part + e;
          const float kv = kn[dd];
#pragma unroll
          for (int h = 0; h < G; ++h) sp[h] += qs[h][dd] * kv;
        }
    } else {
      // q as bf16 pairs from LDS (one 16-byte read per 8 elements, broadcast to the lanes of
      // a key part), two-term bf16 dot products against the raw K words
#pragma unroll
      for (int j = 0; j < KV4; ++j) {
        const uint32_t w4[4] = {kc[j].x, kc[j].y, kc[j].z, kc[j].w};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint4 q4 = *reinterpret_cast<const uint4*>(&qb[h][32 * j + 8 * part]);
          const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sp[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[e]),
                                                    __builtin_bit_cast(bf16x2_t, w4[e]), sp[h], false);
        }
      }
    }
    // next chunk's tiles go out before the softmax and P*V work of this one
    const bool more = t0 + CHW < t_end;
    if (more) load_tiles(kx, vx, t0 + CHW);
    const bool valid = t < t_end;
    // The reference maximum m of a head moves (a wave reduction, and the rescale of o and
    // l) only when a score exceeds it by more than TAU (base 2), so 2^(z - m) <= 2^TAU;
    // otherwise the chunk costs one ballot.  l is kept per lane (its own positions) and
    // summed over the wave once, after the last chunk.
    constexpr float TAU = 12.0f;
    float pr[G], zs[G];
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sp[h] += __shfl_xor(sp[h], 1, 64);
      sp[h] += __shfl_xor(sp[h], 2, 64);
      zs[h] = valid ? sp[h] * scale2 : -INFINITY;
      need = need || (zs[h] > m[h] + TAU);
    }
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mnew = fmaxf(m[h], wave_max(zs[h]));
        const float alpha = (m[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[h] - mnew);
        l[h] *= alpha;
        m[h] = mnew;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pr[h] = valid ? __builtin_amdgcn_exp2f(zs[h] - m[h]) : 0.0f;
      l[h] += part == 0 ? pr[h] : 0.0f;
    }
    // the wave's 16 probabilities per head go through LDS to the P*V lanes (one wave
    // writes and reads its own slots: the fences order the accesses within the wave)
    if (part == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) ps[wid][h][tl] = pr[h];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P*V: each lane its VR positions x 8 dims (position p itself reads zero here and is
    // added from LDS below)
#pragma unroll
    for (int i = 0; i < VR; ++i) {
      const uint32_t w4[4] = {vc[i].x, vc[i].y, vc[i].z, vc[i].w};
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = __uint_as_float(w4[e] << 16);
        vf[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = ps[wid][h][vu + PSL * i];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += pw * vf[e];
      }
    }
    const int pp = p - (t0 + 16 * wid);  // p's place among this wave's positions (uniform)
    if (pp >= 0 && pp < 16 && vu == pp % PSL) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = ps[wid][h][pp];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += pw * vn[8 * vch + e];
      }
    }
    __builtin_amdgcn_wave_barrier();  // ps is rewritten by the next chunk
    if (more) {
#pragma unroll
      for (int j = 0; j < KV4; ++j) kc[j] = kx[j];
#pragma unroll
      for (int i = 0; i < VR; ++i) vc[i] = vx[i];
    }
  }
  // ---- merge the waves' softmax states ----
  // the PSL position slots of each output dim (lanes vch + CL * u) are added first
#pragma unroll
  for (int msk = CL; msk < 64; msk <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[h][e] = msk == 16 ? xor16_sum(o[h][e]) : msk == 32 ? xor32_sum(o[h][e]) : o[h][e] + __shfl_xor(o[h][e], msk, 64);
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = wave_sum(l[h]);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      wm[wid][h] = m[h];
      wl[wid][h] = l[h];
    }
  }
  if (vu == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) wo[wid][h][8 * vch + e] = o[h][e];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (wm[w][h] == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(wm[w][h] - M);
      L += wl[w][h] * f;
      O += wo[w][h][dd] * f;
    }
    const int head = g * G + h;
    if (a.nsplit == 1) {
      a.out[(size_t)b * a.ldo + (size_t)head * D + dd] = f2bf(O / L);
    } else {
      const size_t pi = ((size_t)b * a.H + head) * a.nsplit + s;
      if (a.merge_last == 1) {  // agent-coherent: the merging split reads them without a fence
        __hip_atomic_store(a.part_o + pi * D + dd, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (dd == 0) {
          __hip_atomic_store(a.part_ml + pi * 2, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.part_ml + pi * 2 + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        a.part_o[pi * D + dd] = O;
        if (dd == 0) {
          a.part_ml[pi * 2] = M;
          a.part_ml[pi * 2 + 1] = L;
        }
      }
    }
  }
  if (a.nsplit == 1 || a.merge_last != 1) return;
  // ---- the last split to finish merges all partials of this (row, KV head) ----
  // Each wave's agent-coherent partial stores have completed (s_waitcnt 0) before thread 0
  // counts the split in; the split that counts last reads every partial with
  // agent-coherent loads issued after its count returned, so no cache write-back or
  // invalidate is needed.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned int t = __hip_atomic_fetch_add(a.counters + (size_t)b * a.KV + g, 1u,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (t == (unsigned)a.nsplit - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!last_flag) return;
  // Every split's (max, sum) of the G heads is requested at once; a wave per head turns
  // them into weights 2^(m_s - m) and the total; the outputs are summed over the splits
  // in 16-byte agent-coherent loads, several splits in flight per thread, the split
  // subsets of one output group added through LDS.  A long context (tens of splits)
  // costs two or three memory round trips instead of one per split.
  constexpr int SB = 8;
  if constexpr (!WIDE) {
    // up to SB splits: each thread merges one output from every split's (max, sum,
    // output), all requested at once (one memory round trip, no barrier)
    const int ns = a.nsplit;
    auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    for (int idx = tid; idx < G * D; idx += NT) {
      const int h = idx / D, dd = idx % D;
      const int head = g * G + h;
      const size_t base = ((size_t)b * a.H + head) * ns;
      float mv[SB], lv[SB], ov[SB];
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        mv[k] = k < ns ? ld(a.part_ml + (base + k) * 2) : -INFINITY;
        lv[k] = k < ns ? ld(a.part_ml + (base + k) * 2 + 1) : 0.0f;
        ov[k] = k < ns ? ld(a.part_o + (base + k) * D + dd) : 0.0f;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < SB; ++k) mx = fmaxf(mx, mv[k]);
      float lsum = 0.0f, acc = 0.0f;
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        if (mv[k] == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(mv[k] - mx);
        lsum += lv[k] * w;
        acc += ov[k] * w;
      }
      a.out[(size_t)b * a.ldo + (size_t)head * D + dd] = f2bf(acc / lsum);
    }
  } else {
    __shared__ float mw[G][ATT_MAX_SPLITS], mlv[G][ATT_MAX_SPLITS], hl[G];
    __shared__ f32x4_t redm[NT > G * D / 4 ? NT : G * D / 4];
    const int ns = a.nsplit;
    constexpr int NG4 = G * D / 4;                  // 4-float output groups
    constexpr int SQ = NT >= NG4 ? NT / NG4 : 1;    // split subsets per group
    constexpr int UB = 8;                           // splits in flight per thread
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        a.part_o + ((size_t)b * a.H + (size_t)g * G) * ns * D, 0, G * ns * D * 4, 0x00020000);
    // the first batch of this thread's first output group goes out before the (max, sum)
    // pairs, so a short context (up to SQ * UB splits) costs one memory round trip
    f32x4_t vf[UB];
    {
      const bool ok = tid < NG4 * SQ;
      const int gi = tid % NG4, sq = tid / NG4;
      const int h = (4 * gi) / D, dd = (4 * gi) % D;
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int q = sq + u * SQ;
        vf[u] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                ors, (ok && q < ns) ? ((h * ns + q) * D + dd) * 4 : OOB, 0, 16));
      }
    }
    {
      const size_t base0 = ((size_t)b * a.H + (size_t)g * G) * ns;  // this row's G heads
      for (int i = tid; i < G * ns; i += NT) {
        mw[i / ns][i % ns] = __hip_atomic_load(a.part_ml + (base0 + i) * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mlv[i / ns][i % ns] = __hip_atomic_load(a.part_ml + (base0 + i) * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    for (int h = wid; h < G; h += NW) {
      float mx = -INFINITY;
      for (int q = lane; q < ns; q += 64) mx = fmaxf(mx, mw[h][q]);
      mx = wave_max(mx);
      float ls = 0.0f;
      for (int q = lane; q < ns; q += 64) {
        const float m_s = mw[h][q];
        const float w = m_s == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_s - mx);
        mw[h][q] = w;
        ls += mlv[h][q] * w;
      }
      ls = wave_sum(ls);
      if (lane == 0) hl[h] = ls;
    }
    __syncthreads();
    {
      f32x4_t* red = redm;  // [SQ][NG4]
      for (int e = tid; e < NG4 * SQ; e += NT) {
        const int gi = e % NG4, sq = e / NG4;
        const int h = (4 * gi) / D, dd = (4 * gi) % D;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        int q0 = sq;
        if (e == tid) {  // the batch requested up front
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const int q = sq + u * SQ;
            if (q < ns) acc += vf[u] * mw[h][q];
          }
          q0 += SQ * UB;
        }
        for (; q0 < ns; q0 += SQ * UB) {
          f32x4_t v[UB];
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const int q = q0 + u * SQ;
            v[u] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   ors, q < ns ? ((h * ns + q) * D + dd) * 4 : OOB, 0, 16));
          }
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const int q = q0 + u * SQ;
            if (q < ns) acc += v[u] * mw[h][q];
          }
        }
        red[sq * NG4 + gi] = acc;
      }
      __syncthreads();
      for (int gi = tid; gi < NG4; gi += NT) {
        f32x4_t acc = red[gi];
        for (int sq = 1; sq < SQ; ++sq) acc += red[sq * NG4 + gi];
        const int h = (4 * gi) / D, dd = (4 * gi) % D;
        const float lh = hl[h];
        bf16_t* o = a.out + (size_t)b * a.ldo + (size_t)(g * G + h) * D + dd;
        const uint32_t lo = (uint32_t)f2bf(acc[0] / lh) | ((uint32_t)f2bf(acc[1] / lh) << 16);
        const uint32_t hi = (uint32_t)f2bf(acc[2] / lh) | ((uint32_t)f2bf(acc[3] / lh) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
      }
    }
  }
  if (tid == 0) __hip_atomic_store(a.counters + (size_t)b * a.KV + g, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
}

// split merge as its own launch: o = sum_s o_s 2^(m_s - m) / sum_s l_s 2^(m_s - m) (the
// splits' maxima are in base 2)
// for one (row b, query head); the kernel boundary orders it after every split.  All
// (max, sum) pairs and the first eight splits' partials are requested at once, so a short
// context costs one memory round trip.
__global__ __launch_bounds__(128) void k_attn_dec_merge(AttnDecArgs a) {
  __shared__ float wsp[ATT_MAX_SPLITS];  // 2^(m_s - m), zero for an empty split
  __shared__ float red[2];
  constexpr int SB = 8;
  const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int ns = a.nsplit, D = a.D;
  const size_t base = ((size_t)b * a.H + head) * ns;
  float ov[2][SB];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int dd = tid + 128 * k;
#pragma unroll
    for (int s = 0; s < SB; ++s) ov[k][s] = (dd < D && s < ns) ? a.part_o[(base + s) * D + dd] : 0.0f;
  }
  float m0 = -INFINITY, l0 = 0.0f, m1 = -INFINITY, l1 = 0.0f;
  if (tid < ns) {
    m0 = a.part_ml[(base + tid) * 2];
    l0 = a.part_ml[(base + tid) * 2 + 1];
  }
  if (tid + 128 < ns) {
    m1 = a.part_ml[(base + tid + 128) * 2];
    l1 = a.part_ml[(base + tid + 128) * 2 + 1];
  }
  float mx = wave_max(fmaxf(m0, m1));
  if (lane == 0) red[wid] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  const float f0 = m0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m0 - mx);
  const float f1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
  if (tid < ns) wsp[tid] = f0;
  if (tid + 128 < ns) wsp[tid + 128] = f1;
  float ls = wave_sum(l0 * f0 + l1 * f1);
  __syncthreads();
  if (lane == 0) red[wid] = ls;
  __syncthreads();
  const float lsum = red[0] + red[1];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int dd = tid + 128 * k;
    if (dd >= D) continue;
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < SB; ++s)
      if (s < ns) acc += ov[k][s] * wsp[s];
    for (int s0 = SB; s0 < ns; s0 += SB) {
      float v[SB];
#pragma unroll
      for (int s = 0; s < SB; ++s) v[s] = s0 + s < ns ? a.part_o[(base + s0 + s) * D + dd] : 0.0f;
#pragma unroll
      for (int s = 0; s < SB; ++s)
        if (s0 + s < ns) acc += v[s] * wsp[s0 + s];
    }
    a.out[(size_t)b * a.ldo + (size_t)head * D + dd] = f2bf(acc / lsum);
  }
}

// ------------------------------------------------------------------------------------------
// Prefill attention on MFMA (causal, flash style).  A work-group owns up to 64*RG query
// rows of one sequence (4 waves x RG groups of 16 rows: wave w holds rows 64*rg + 16*w ..)
// and one query head h of KV group g = h / (H/KV).  With RG = 2 every K and V fragment read
// from LDS feeds two row groups' MFMAs (half the LDS reads per score), at 2 work-groups
// per CU instead of 3; long prompts take it, short ones keep RG = 1 for more work-groups.
// Keys and values advance in blocks of 64 positions staged once in LDS for all waves
// (V transposed).  Each wave computes the transposed products S^T = K Q^T and
// O^T = V^T P^T, so a lane always holds one query row (its lane index mod 16): the MFMA
// output layout of S^T is then already the B-operand layout P^T needs, P never leaves
// registers, and a row's softmax state is one scalar per lane.  For that, the 16 rows of
// the S^T tile t of a 32-key step are keys 8*(r/4) + 4t + r%4; K rows are stored in LDS in
// that order (key 8a + 4t + i of a 32-key step at row 16t + 4a + i), so the fragment reads
// stay on consecutive rows.  P is split into bf16 high and low parts (two MFMAs), so the
// probabilities enter the product with ~16 significant bits rather than bf16's 8.
template <int D, int RG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 4 - RG : 1))) void k_flash_prefill(
    QD_FLASH_PRELOAD_PARAMS, FlashArgs a) {
  QD_FLASH_PRELOAD_SET(a);
  constexpr int KB = 64;             // keys per block
  constexpr int NKK = KB / 32;       // 32-key steps per block (two S^T tiles each)
  constexpr int KS = D / 32;         // MFMA k-steps over the head dim
  constexpr int NT = D / 16;         // 16-dim tiles of O^T
  constexpr int VPR = D / 8;         // uint4 per key row
  constexpr int LD_PER_T = (KB * VPR + 255) / 256;  // uint4 per thread per tensor and block
  __shared__ __align__(16) bf16_t Ks[KB][D + 8];
  __shared__ __align__(16) bf16_t Vt[D][KB + 8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = lane >> 4, r16 = lane & 15;
  // heads vary fastest and tiles run last to first: within a sequence later tiles see more
  // keys, so the longest work-groups start first and the shortest fill the end of the grid
  const int4 tile = a.tiles[gridDim.y - 1 - blockIdx.y];
  const int row0 = tile.x, slot = tile.y, pos0 = tile.z, nrows = tile.w;
  const int h = blockIdx.x, G = a.H / a.KV, g = h / G;
  const bf16_t* Kb = a.kcache + ((size_t)slot * a.KV + g) * a.max_ctx * D;
  const bf16_t* Vb = a.vcache + ((size_t)slot * a.KV + g) * a.max_ctx * D;
  const int kmax = pos0 + nrows;  // keys 0..kmax-1 are visible to some row of the tile

  // this lane's query rows (one per row group) and their Q fragments (B operand of S^T):
  // dims 32*ks + 8*grp
  int r[RG], qpos[RG];
  bool row_ok[RG];
  bf16x8_t qf[RG][KS];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    r[rg] = 64 * rg + 16 * wid + r16;
    row_ok[rg] = r[rg] < nrows;
    qpos[rg] = pos0 + r[rg];
    const bf16_t* qr = a.q + (size_t)(row0 + (row_ok[rg] ? r[rg] : 0)) * a.ldq + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[rg][ks] = __builtin_bit_cast(
          bf16x8_t, row_ok[rg] ? *reinterpret_cast<const uint4*>(qr + 32 * ks + 8 * grp) : make_uint4(0, 0, 0, 0));
  }
  // softmax state of the lane's rows: m is the same in a row's four lanes (reduced), l is
  // this lane's share of the row sum (its keys only), reduced once at the end
  float m[RG], l[RG];
  f32x4_t o[RG][NT];  // O^T: dims 16*nt + 4*grp + i of the lane's rows
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m[rg] = -INFINITY;
    l[rg] = 0.0f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[rg][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // scores in base 2: exp(z - m) = exp2(z*log2(e) - m*log2(e)), one hardware exp each
  const float scale2 = 1.4426950408889634f / sqrtf((float)D);

  // global -> register staging of the next K/V block while this one is in use (one
  // register set, so three work-groups fit on a CU at head dim 128).  K: consecutive
  // lanes take consecutive 16-byte pieces of a key row.  V: consecutive lanes take
  // consecutive key pairs (same piece), so the transposed LDS stores of half a wave hit
  // consecutive words instead of rows 8 apart (which all map to one bank).  Buffer
  // loads: keys past the tile's last visible one read zero through an out-of-range
  // offset, so no load sits in a branch and each block waits only for its own data.
  constexpr int OOB = (int)0x80000000;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kb, 0, a.max_ctx * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vb, 0, a.max_ctx * D * 2, 0x00020000);
  // V in units of (key pair, 16-byte piece): the transposed LDS stores write both keys of
  // a dim as one 32-bit word
  constexpr int NVU = KB / 2 * VPR;
  constexpr int VPT = (NVU + 255) / 256;  // V units per thread and block
  uint4 kst[LD_PER_T], vst[VPT][2];
  auto fetch = [&](int kb, uint4 (&ks)[LD_PER_T], uint4 (&vs)[VPT][2]) {
#pragma unroll
    for (int u = 0; u < LD_PER_T; ++u) {
      const int idx = tid + 256 * u;
      const int key = idx / VPR, c = idx % VPR;
      const bool in = idx < KB * VPR;
      ks[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            krs, (in && kb + key < kmax) ? ((kb + key) * D + 8 * c) * 2 : OOB, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int pidx = tid + 256 * u;
      const int kp = pidx % (KB / 2), vc = pidx / (KB / 2);
      const bool in = pidx < NVU;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int vkey = kb + 2 * kp + j;
        vs[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 vrs, (in && vkey < kmax) ? (vkey * D + 8 * vc) * 2 : OOB, 0, 0));
      }
    }
  };
  // one key block: stage it in LDS, refill the registers with the next block, then
  // S^T = K Q^T, online softmax, O^T += V^T P^T
  // FULL: every key of the block precedes every row of the tile (no causal mask to apply;
  // rows past the tile's end hold zero queries whose finite results are never stored)
  auto block = [&](auto full, int kb, uint4 (&ks)[LD_PER_T], uint4 (&vs)[VPT][2]) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int u = 0; u < LD_PER_T; ++u) {
      const int idx = tid + 256 * u;
      if (idx < KB * VPR) {
        const int key = idx / VPR, c = idx % VPR;
        const int kq = key & 31;  // 8a + 4t + i -> row 16t + 4a + i of its 32-key step
        const int krow = (key & ~31) + 16 * ((kq >> 2) & 1) + 4 * (kq >> 3) + (kq & 3);
        *reinterpret_cast<uint4*>(&Ks[krow][8 * c]) = ks[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int pidx = tid + 256 * u;
      if (pidx < NVU) {
        const int kp = pidx % (KB / 2), vc = pidx / (KB / 2);
        const uint32_t a4[4] = {vs[u][0].x, vs[u][0].y, vs[u][0].z, vs[u][0].w};
        const uint32_t b4[4] = {vs[u][1].x, vs[u][1].y, vs[u][1].z, vs[u][1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<uint32_t*>(&Vt[8 * vc + 2 * e][2 * kp]) = (a4[e] & 0xFFFFu) | (b4[e] << 16);
          *reinterpret_cast<uint32_t*>(&Vt[8 * vc + 2 * e + 1][2 * kp]) = (a4[e] >> 16) | (b4[e] & 0xFFFF0000u);
        }
      }
    }
    __syncthreads();
    fetch(kb + KB, ks, vs);  // past kmax: reads zero, never used

    // S^T tiles: st[rg][kk][t][i] = score of the lane's row of group rg against key
    // kb + 32kk + 8grp + 4t + i (each K fragment read feeds the RG row groups)
    f32x4_t st[RG][NKK][2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) st[rg][kk][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks2 = 0; ks2 < KS; ++ks2) {
          const bf16x8_t kf = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4*>(&Ks[32 * kk + 16 * t + r16][32 * ks2 + 8 * grp]));
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            st[rg][kk][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rg][ks2], st[rg][kk][t], 0, 0, 0);
        }
      }
    // causal mask + online softmax.  The row's reference maximum m moves only when the
    // block's maximum exceeds it by more than 2^TAU (so probabilities stay below 2^TAU);
    // the wave rescales O only then (the result is the same softmax, any reference gives it).
    // The maximum is taken over the raw scores (the scale is positive, so the scaled maximum
    // is the maximum scaled), and each weight is 2^(s * scale2 - m) from one fused
    // multiply-add.
    constexpr float TAU = 8.0f;
    // P^T fragments (B operand): keys 32kk + 8grp + j, j = 4t + i.  p = hi + lo exactly,
    // hi = p with its low 16 bits cleared (a bf16 value), lo = p - hi rounded to bf16, so the
    // probabilities enter the product with ~16 significant bits rather than bf16's 8.
    bf16x8_t phi[RG][NKK], plo[RG][NKK];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      float sv[NKK][2][4];
      float smax = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb + 32 * kk + 8 * grp + 4 * t + i;
            sv[kk][t][i] = (FULL || (row_ok[rg] && key <= qpos[rg])) ? st[rg][kk][t][i] : -INFINITY;
            smax = fmaxf(smax, sv[kk][t][i]);
          }
      smax = xor32_max(xor16_max(smax)) * scale2;
      if (__any(smax > m[rg] + TAU)) {
        const float mnew = fmaxf(m[rg], smax);
        const float alpha = (m[rg] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[rg] - mnew);
        l[rg] *= alpha;
        m[rg] = mnew;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rg][nt][i] *= alpha;
      }
      const float negm = -m[rg];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          float pv[2], lo[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 2 * j2 + e, t = j >> 2, i = j & 3;
            const float p = (!FULL && sv[kk][t][i] == -INFINITY)
                                ? 0.0f
                                : __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kk][t][i], scale2, negm));
            l[rg] += p;
            pv[e] = p;
            lo[e] = p - __uint_as_float(__float_as_uint(p) & 0xFFFF0000u);
          }
          hw[j2] = __builtin_amdgcn_perm(__float_as_uint(pv[1]), __float_as_uint(pv[0]), 0x07060302u);
          lw[j2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo[0], lo[1]}, bf16x2_t));
        }
        phi[rg][kk] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        plo[rg][kk] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
    }
    // O^T += V^T P^T: A = V^T (dims 16nt + r16, keys 32kk + 8grp..), B = P^T
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&Vt[16 * nt + r16][32 * kk + 8 * grp]));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          o[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[rg][kk], o[rg][nt], 0, 0, 0);
          o[rg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[rg][kk], o[rg][nt], 0, 0, 0);
        }
      }
    __syncthreads();
  };
  fetch(0, kst, vst);
  const int kfull = min(kmax, (pos0 + 1) / KB * KB);
  int kb = 0;
  for (; kb < kfull; kb += KB) block(std::true_type{}, kb, kst, vst);
  for (; kb < kmax; kb += KB) block(std::false_type{}, kb, kst, vst);
  // each row sum over its four lanes; out[r][h*D + 16nt + 4grp + i], four dims per store
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    float lr = l[rg];
    lr = xor32_sum(xor16_sum(lr));
    if (!row_ok[rg]) continue;
    bf16_t* orow = a.out + (size_t)(row0 + r[rg]) * a.ldo + (size_t)h * D + 4 * grp;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t w0 = (uint32_t)f2bf(o[rg][nt][0] / lr) | ((uint32_t)f2bf(o[rg][nt][1] / lr) << 16);
      const uint32_t w1 = (uint32_t)f2bf(o[rg][nt][2] / lr) | ((uint32_t)f2bf(o[rg][nt][3] / lr) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * nt) = make_uint2(w0, w1);
    }
  }
}

// ------------------------------------------------------------------------------------------
// launchers

hipError_t launch_quantize_rows(const float* w, int rows, int cols, int8_t* q, float* s,
                                int dst_row0, int gu_half, hipStream_t st) {
  hipLaunchKernelGGL(k_quantize_rows, dim3(rows), dim3(256), 0, st, w, cols, q, s, dst_row0,
                     gu_half);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int max_ctx, int D, float theta, hipStream_t st) {
  const long n = (long)max_ctx * (D / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab,
                     max_ctx, D, (double)theta);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}


hipError_t launch_set_positions(int* pos, const int* lens, const int* slots, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_set_positions, dim3((n + 255) / 256), dim3(256), 0, st, pos, lens, slots, n);
  return hipGetLastError();
}

hipError_t launch_iota(int* p, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_iota, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_embed(const int* ids, int M, const int8_t* E, const float* Es, int d, int V,
                        bf16_t* x, hipStream_t st, int* counts, const int* row_slot) {
  if (d % 4 || d > 8192) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, ids, E, Es, d, V, x, counts, row_slot);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const bf16_t* x, int M, int d, const float* g, float eps, bf16_t* y,
                          hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if ((d & 7) || d > 8192) return hipErrorInvalidValue;
  const int cpl = (d / 8 + 63) / 64;  // 16-byte chunks per lane
  dim3 grid((M + 3) / 4), blk(256);
  if (cpl <= 1) hipLaunchKernelGGL(k_rmsnorm<1>, grid, blk, 0, st, x, M, d, g, eps, y);
  else if (cpl <= 2) hipLaunchKernelGGL(k_rmsnorm<2>, grid, blk, 0, st, x, M, d, g, eps, y);
  else if (cpl <= 4) hipLaunchKernelGGL(k_rmsnorm<4>, grid, blk, 0, st, x, M, d, g, eps, y);
  else if (cpl <= 8) hipLaunchKernelGGL(k_rmsnorm<8>, grid, blk, 0, st, x, M, d, g, eps, y);
  else hipLaunchKernelGGL(k_rmsnorm<16>, grid, blk, 0, st, x, M, d, g, eps, y);
  return hipGetLastError();
}

template <int S>
static hipError_t resid_norm_s(bf16_t* x, int M, int d, const float* part, const float* scale,
                               const float* g, float eps, bf16_t* y, hipStream_t st) {
  const int cpl = (d / 8 + 63) / 64;  // 16-byte chunks per lane
  dim3 grid((M + 3) / 4), blk(256);
  if (cpl <= 1) hipLaunchKernelGGL((k_resid_norm<1, S>), grid, blk, 0, st, x, M, d, part, scale, g, eps, y);
  else if (cpl <= 2) hipLaunchKernelGGL((k_resid_norm<2, S>), grid, blk, 0, st, x, M, d, part, scale, g, eps, y);
  else if (cpl <= 4) hipLaunchKernelGGL((k_resid_norm<4, S>), grid, blk, 0, st, x, M, d, part, scale, g, eps, y);
  else if (cpl <= 8) hipLaunchKernelGGL((k_resid_norm<8, S>), grid, blk, 0, st, x, M, d, part, scale, g, eps, y);
  else hipLaunchKernelGGL((k_resid_norm<16, S>), grid, blk, 0, st, x, M, d, part, scale, g, eps, y);
  return hipGetLastError();
}

hipError_t launch_resid_norm(bf16_t* x, int M, int d, const float* part, int splits,
                             const float* scale, const float* g, float eps, bf16_t* y,
                             hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if ((d & 7) || d > 8192) return hipErrorInvalidValue;
  switch (splits) {
    case 2: return resid_norm_s<2>(x, M, d, part, scale, g, eps, y, st);
    case 4: return resid_norm_s<4>(x, M, d, part, scale, g, eps, y, st);
    case 8: return resid_norm_s<8>(x, M, d, part, scale, g, eps, y, st);
    default: return hipErrorInvalidValue;
  }
}

template <int R, int KC>
static hipError_t gemv1_rk(const GemvArgs& a, int epi, hipStream_t st) {
  const int nout = epi == EPI_SILU ? a.N / 2 : a.N;
  const int nblk = (nout + 4 * R - 1) / (4 * R);
  dim3 grid(epi == EPI_LOGITS ? (nblk < LM_MAX_GRID ? nblk : LM_MAX_GRID) : nblk);
  // the leading (preloaded) arguments: see k_gemv1
  const void* xp = a.x;
  const void* gp = a.gain;
  const void* rp = a.x_rows;
#define QD_GEMV1(E, M, P0, P1, I0, I1)                                                            \
  hipLaunchKernelGGL((k_gemv1<R, KC, E, M>), grid, dim3(256), 0, st, a.W, a.scale, P0, P1, rp, a.N, \
                     a.K, I0, I1, a)
  switch (epi) {
    case EPI_STORE: QD_GEMV1(EPI_STORE, false, xp, gp, a.ldx, 0); break;
    case EPI_RESID:
      if (a.att_ns > 0) {
        if (a.att_ns > ATT_DEFER_MAX_SPLITS || a.att_D <= 0 || a.att_D % 8 || a.K % a.att_D || !a.att_po ||
            !a.att_ml || a.K > 64 * 16 * KC)
          return hipErrorInvalidValue;
        QD_GEMV1(EPI_RESID, true, static_cast<const void*>(a.att_po), static_cast<const void*>(a.att_ml),
                 a.att_ns, a.att_D);
      } else {
        QD_GEMV1(EPI_RESID, false, xp, gp, a.ldx, 0);
      }
      break;
    case EPI_SILU: QD_GEMV1(EPI_SILU, false, xp, gp, a.ldx, 0); break;
    default: QD_GEMV1(EPI_LOGITS, false, xp, gp, a.ldx, 0); break;
  }
#undef QD_GEMV1
  return hipGetLastError();
}

template <int R>
static hipError_t gemv1_r(const GemvArgs& a, int epi, hipStream_t st) {
  const int kc = (a.K + 1023) / 1024;
  switch (kc) {
    case 1: return gemv1_rk<R, 1>(a, epi, st);
    case 2: return gemv1_rk<R, 2>(a, epi, st);
    case 3: return gemv1_rk<R, 3>(a, epi, st);
    case 4: return gemv1_rk<R, 4>(a, epi, st);
    case 5: case 6: return gemv1_rk<R, 6>(a, epi, st);
    default: return gemv1_rk<R, 8>(a, epi, st);
  }
}

// one row: register kernel; enough work-groups per matrix to cover the GPU
static hipError_t gemv1(const GemvArgs& a, int epi, hipStream_t st) {
  if (a.K > 8192) return hipErrorInvalidValue;
  const int nout = epi == EPI_SILU ? a.N / 2 : a.N;
  // rows per wave: 2 for the q|k|v projection of a 1024-wide model (512 work-groups; 1 and 4
  // rows measured slower), 4 for the LM head and other wide projections, else 1
  if (epi == EPI_STORE && nout >= 4096 && a.K <= 1024) return gemv1_rk<2, 1>(a, epi, st);
  if ((epi == EPI_LOGITS || nout >= 4096) && a.K <= 2048)
    return a.K <= 1024 ? gemv1_rk<4, 1>(a, epi, st) : gemv1_rk<4, 2>(a, epi, st);
  return gemv1_r<1>(a, epi, st);
}

static hipError_t lm_finish(const GemvArgs& a, int nblocks, hipStream_t st) {
  hipLaunchKernelGGL(k_lm_finish, dim3(a.nb), dim3(256), 0, st, a.part_keys, a.next_ids, a.pos, a.row_slot,
                     a.out_ids, a.step, nblocks, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.bump_step || a.nb == 1) return e;
  hipLaunchKernelGGL(k_lm_finish_step, dim3(1), dim3(1), 0, st, a.step);
  return hipGetLastError();
}

// one row only; batches go through launch_skinny
hipError_t launch_gemv(const GemvArgs& a, int epi, hipStream_t st) {
  if (a.nb != 1) return hipErrorInvalidValue;
  hipError_t e = gemv1(a, epi, st);
  if (e != hipSuccess || epi != EPI_LOGITS) return e;
  const int nblk = (a.N + 15) / 16;
  return lm_finish(a, nblk < LM_MAX_GRID ? nblk : LM_MAX_GRID, st);
}

// XS: activations through row-contiguous loads and a per-wave LDS slot
template <int TT, bool XS = false>
static hipError_t skinny_tt(const GemvArgs& a, int epi, hipStream_t st) {
  if (epi == EPI_LOGITS) {
    // vocabulary-sized: 4 x LMT wave tiles per work-group, activations staged in LDS
    const int ntiles = (a.N + 15) / 16;
    const int g = (ntiles + 4 * LMT - 1) / (4 * LMT);
    if (g > LM_MAX_GRID || (a.K & 31) || (size_t)a.N * a.K > 0x7FFFFFFFu) return hipErrorInvalidValue;
    if (a.K == 1024) hipLaunchKernelGGL((k_lm_skinny<TT, 8>), dim3(g), dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
    else if (a.K == 2048) hipLaunchKernelGGL((k_lm_skinny<TT, 16>), dim3(g), dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
    else hipLaunchKernelGGL((k_lm_skinny<TT, 0>), dim3(g), dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
    hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : lm_finish(a, g, st);
  }
  const int ctw = epi == EPI_SILU ? 2 : 1;
  const int ntiles = (a.N + 16 * ctw - 1) / (16 * ctw);
  if (a.ksplit > 1) {
    if (ntiles > SKINNY_MAX_TILES || a.ksplit > SKINNY_MAX_SPLIT ||
        (size_t)ntiles * a.ksplit * ctw * TT * 256 > GEMM_PART_FLOATS || !a.kpart || !a.kcnt)
      return hipErrorInvalidValue;
    dim3 g(ntiles * a.ksplit);
    if (XS) {
      switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL((k_skinny_split<TT, EPI_STORE, 4, XS>), g, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        case EPI_RESID: hipLaunchKernelGGL((k_skinny_split<TT, EPI_RESID, 4, XS>), g, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        default: hipLaunchKernelGGL((k_skinny_split<TT, EPI_SILU, 4, XS>), g, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      }
    } else {
      switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL((k_skinny_split<TT, EPI_STORE, 4>), g, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        case EPI_RESID: hipLaunchKernelGGL((k_skinny_split<TT, EPI_RESID, 4>), g, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        default: hipLaunchKernelGGL((k_skinny_split<TT, EPI_SILU, 4>), g, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      }
    }
    return hipGetLastError();
  }
  dim3 grid(ntiles);
  if (ntiles < 128) {  // few tiles: eight waves split K eight ways
    if (XS) {
      switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL((k_skinny<TT, EPI_STORE, 8, XS>), grid, dim3(512), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        case EPI_RESID: hipLaunchKernelGGL((k_skinny<TT, EPI_RESID, 8, XS>), grid, dim3(512), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        default: hipLaunchKernelGGL((k_skinny<TT, EPI_SILU, 8, XS>), grid, dim3(512), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      }
    } else {
      switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL((k_skinny<TT, EPI_STORE, 8>), grid, dim3(512), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        case EPI_RESID: hipLaunchKernelGGL((k_skinny<TT, EPI_RESID, 8>), grid, dim3(512), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
        default: hipLaunchKernelGGL((k_skinny<TT, EPI_SILU, 8>), grid, dim3(512), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      }
    }
  } else if (XS) {
    switch (epi) {
      case EPI_STORE: hipLaunchKernelGGL((k_skinny<TT, EPI_STORE, 4, XS>), grid, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      case EPI_RESID: hipLaunchKernelGGL((k_skinny<TT, EPI_RESID, 4, XS>), grid, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      default: hipLaunchKernelGGL((k_skinny<TT, EPI_SILU, 4, XS>), grid, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
    }
  } else {
    switch (epi) {
      case EPI_STORE: hipLaunchKernelGGL((k_skinny<TT, EPI_STORE, 4>), grid, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      case EPI_RESID: hipLaunchKernelGGL((k_skinny<TT, EPI_RESID, 4>), grid, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
      default: hipLaunchKernelGGL((k_skinny<TT, EPI_SILU, 4>), grid, dim3(256), 0, st, QD_SKINNY_PRELOAD_ARGS(a), a); break;
    }
  }
  return hipGetLastError();
}

template <int TT, int NB>
static hipError_t skinny_norm_launch(const GemvArgs& a, int epi, hipStream_t st) {
  const int ctw = epi == EPI_SILU ? 2 : 1;
  dim3 grid((a.N + 16 * ctw - 1) / (16 * ctw)), blk(64 * SKN_WAVES);
  // row-contiguous staging above 8 rows (measured per step: B = 32 +2.0%, B = 16 +0.9%,
  // B = 8 -0.7%)
  if (!a.no_xstage && a.nb > 8) {
    if (epi == EPI_STORE) hipLaunchKernelGGL((k_skinny_norm<TT, EPI_STORE, NB, true>), grid, blk, 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
    else hipLaunchKernelGGL((k_skinny_norm<TT, EPI_SILU, NB, true>), grid, blk, 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
  } else {
    if (epi == EPI_STORE) hipLaunchKernelGGL((k_skinny_norm<TT, EPI_STORE, NB>), grid, blk, 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
    else hipLaunchKernelGGL((k_skinny_norm<TT, EPI_SILU, NB>), grid, blk, 0, st, QD_SKINNY_PRELOAD_ARGS(a), a);
  }
  return hipGetLastError();
}

// the shapes whose folded-norm kernel keeps every block in registers without spilling:
// one 16-token tile with up to 4 blocks per wave, two tiles with up to 2
bool skinny_norm_ok(int nb, int K, int epi, int ksplit) {
  if (nb < 2 || nb > 32 || (K & 127) || K <= 0 || ksplit > 1) return false;
  if (epi != EPI_STORE && epi != EPI_SILU) return false;
  const int blocks = (K + 128 * SKN_WAVES - 1) / (128 * SKN_WAVES);
  return nb <= 16 ? blocks <= 4 : blocks <= 2;
}

// 2..64 token rows.  gain NULL: activations already normalized.  gain set: pre-norm
// activations, RMSNorm folded in (shapes skinny_norm_ok accepts)
hipError_t launch_skinny(const GemvArgs& a, int epi, hipStream_t st) {
  if (a.nb < 1 || a.nb > 64 || (a.K & 31)) return hipErrorInvalidValue;
  if (a.gain) {
    if (!skinny_norm_ok(a.nb, a.K, epi, a.ksplit)) return hipErrorInvalidValue;
    const int blocks = (a.K + 128 * SKN_WAVES - 1) / (128 * SKN_WAVES);
    if (a.nb > 16) return skinny_norm_launch<2, 2>(a, epi, st);
    return blocks <= 2 ? skinny_norm_launch<1, 2>(a, epi, st) : skinny_norm_launch<1, 4>(a, epi, st);
  }
  // row-contiguous activation staging for one 16-row tile (measured: B = 8 and 16 gain
  // 4-5% per layer; two tiles at B = 32 lose 1.4% in the split O and down projections)
  if (a.nb <= 16) return a.no_xstage ? skinny_tt<1>(a, epi, st) : skinny_tt<1, true>(a, epi, st);
  if (a.nb <= 32) return skinny_tt<2>(a, epi, st);
  return skinny_tt<4>(a, epi, st);
}

hipError_t launch_gemm(const GemmArgs& a0, hipStream_t st, int* splits_used, int* rope_done) {
  GemmArgs a = a0;
  if (rope_done) *rope_done = 0;
  if ((a.K & 31) || (size_t)(a.M + 64) * a.lda * 2 > 0x7FFFFFFFu || (size_t)(a.N + 64) * a.K > 0x7FFFFFFFu ||
      (size_t)(a.M + 64) * a.ldo * 2 > 0x7FFFFFFFu)
    return hipErrorInvalidValue;
  // q|k|v and gate/up at many token rows: 256x256 tiles with operands loaded straight into
  // LDS, when they alone give every CU a tile (K a multiple of 64)
  const int dl_tiles = ((a.N + 255) / 256) * ((a.M + 255) / 256);
  // (q|k|v only with its QK-norm / RoPE epilogue, at head dim 128: two heads per tile)
  const bool dl_qkv = a.epi == EPI_STORE && a.fuse_rope && a.rope.D == 128 &&
                      a.N == (a.rope.H + 2 * a.rope.KV) * a.rope.D && a.rope.M == a.M;
  // (gate/up: its outputs are stored as 16-byte pieces, 8 per row piece)
  const bool dl_silu = a.epi == EPI_SILU && a.N % 16 == 0 && a.ldo % 8 == 0;
  if (dl_tiles >= 256 && a.use_big != 0 && (dl_silu || dl_qkv) && a.K % 64 == 0 && a.lda % 8 == 0) {
    if (splits_used) *splits_used = 1;
    if (a.epi == EPI_SILU) {
      a.fuse_rope = 0;
      hipLaunchKernelGGL((k_gemm_dl<EPI_SILU, 2>), dim3(dl_tiles), dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a);
    } else {
      if (rope_done) *rope_done = 1;
      hipLaunchKernelGGL((k_gemm_dl<EPI_STORE, 2>), dim3(dl_tiles), dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a);
    }
    return hipGetLastError();
  }
  // the residual projections (O, down) at many token rows: 256x128 tiles, same loads
  const int dl_tiles_n = ((a.N + 127) / 128) * ((a.M + 255) / 256);
  const bool resid_pieces = a.N % 8 == 0 && a.ldo % 8 == 0;  // 16-byte residual updates
  if (dl_tiles_n >= 256 && a.use_big != 0 && a.epi == EPI_RESID && a.K % 64 == 0 && a.lda % 8 == 0 &&
      resid_pieces) {
    if (splits_used) *splits_used = 1;
    hipLaunchKernelGGL((k_gemm_dl<EPI_RESID, 4>), dim3(dl_tiles_n), dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a);
    return hipGetLastError();
  }
  // many token rows: 128x128 tiles when they alone give every CU at least one
  const int big_tiles = ((a.N + 127) / 128) * ((a.M + 127) / 128);
  if (big_tiles >= 256 && a.use_big != 0 && (a.epi != EPI_RESID || resid_pieces)) {
    if (splits_used) *splits_used = 1;
    const RopeArgs& r = a.rope;
    a.fuse_rope = a.fuse_rope && a.epi == EPI_STORE && (r.D == 64 || r.D == 128) &&
                  a.N == (r.H + 2 * r.KV) * r.D && a.ldo % 4 == 0 && r.M == a.M;
    if (rope_done) *rope_done = a.fuse_rope;
    switch (a.epi) {
      case EPI_STORE: hipLaunchKernelGGL(k_gemm_big<EPI_STORE>, dim3(big_tiles), dim3(256), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;
      case EPI_RESID: hipLaunchKernelGGL(k_gemm_big<EPI_RESID>, dim3(big_tiles), dim3(256), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;
      default: hipLaunchKernelGGL(k_gemm_big<EPI_SILU>, dim3(big_tiles), dim3(256), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;
    }
    return hipGetLastError();
  }
  const bool want_rope = a.fuse_rope != 0;
  a.fuse_rope = 0;
  const int tiles = ((a.N + 63) / 64) * ((a.M + 63) / 64);
  // few rows (at most two 64-row tiles): the k-sliced kernel when its k splits (256..1024 k
  // each) cover K; more than one split only as deferred residual partials, enough splits to
  // give every CU a tile.  Its operand fragments come straight from memory in MFMA lane
  // order (16 rows per instruction), which streams slower than the staged kernel's row-
  // contiguous loads once the tiles re-read enough of A: measured faster at 16 and 100 rows,
  // slower from 256 rows up.
  if (a.use_ks != 0 && a.M <= 128) {
    int S = 1;
    const bool part_ok = a.defer && a.epi == EPI_RESID && a.part;
    if (part_ok)
      while (S < 8 && (tiles * S < 256 || a.K > S * 1024) && a.K >= S * 2 * 256 &&
             (size_t)(S * 2) * a.M * a.N <= GEMM_PART_FLOATS)
        S *= 2;
    const int C = (a.K + S * 256 - 1) / (S * 256);
    if (C <= 4 && (S == 1 || part_ok)) {
      a.splits = S;
      if (splits_used) *splits_used = S;
      dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, S);
      const int epi = S > 1 ? (int)EPI_PART : a.epi;
#define QD_KS(E)                                                                                   \
  switch (C) {                                                                                     \
    case 1: hipLaunchKernelGGL((k_gemm_ks<E, 1>), grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;               \
    case 2: hipLaunchKernelGGL((k_gemm_ks<E, 2>), grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;               \
    case 3: hipLaunchKernelGGL((k_gemm_ks<E, 3>), grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;               \
    default: hipLaunchKernelGGL((k_gemm_ks<E, 4>), grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;              \
  }
      switch (epi) {
        case EPI_STORE: QD_KS(EPI_STORE) break;
        case EPI_RESID: QD_KS(EPI_RESID) break;
        case EPI_PART: QD_KS(EPI_PART) break;
        default: QD_KS(EPI_SILU) break;
      }
#undef QD_KS
      return hipGetLastError();
    }
  }
  // q|k|v with its QK-norm / RoPE epilogue at more rows than the k-sliced kernel took:
  // 32x128 tiles, each holding whole heads
  {
    const RopeArgs& r = a.rope;
    if (want_rope && a.epi == EPI_STORE && (r.D == 64 || r.D == 128) && a.N % 128 == 0 &&
        a.N == (r.H + 2 * r.KV) * r.D && a.ldo % 4 == 0 && r.M == a.M) {
      a.fuse_rope = 1;
      if (splits_used) *splits_used = 1;
      if (rope_done) *rope_done = 1;
      hipLaunchKernelGGL(k_gemm_qr, dim3(a.N / 128, (a.M + 31) / 32), dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a);
      return hipGetLastError();
    }
  }
  // split K when the tile grid leaves most of the 256 CUs idle
  int splits = 1;
  const int max_splits = a.splits > 0 ? a.splits : 8;  // caller's cap (tuning), else 8
  while (splits < max_splits && tiles * splits < 256 && a.K / (splits * 2) >= 256 &&
         (size_t)(splits * 2) * tiles * 4096 <= GEMM_PART_FLOATS && a.part && a.cnt &&
         tiles <= SKINNY_MAX_TILES)
    splits *= 2;
  a.splits = splits;
  if (splits_used) *splits_used = splits;
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, splits);
  if (a.defer && a.epi == EPI_RESID && splits > 1) {
    if ((size_t)splits * a.M * a.N > GEMM_PART_FLOATS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gemm<EPI_PART>, grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a);
    return hipGetLastError();
  }
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL(k_gemm<EPI_STORE>, grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;
    case EPI_RESID: hipLaunchKernelGGL(k_gemm<EPI_RESID>, grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;
    default: hipLaunchKernelGGL(k_gemm<EPI_SILU>, grid, dim3(512), 0, st, QD_GEMM_PRELOAD_ARGS(a), a); break;
  }
  return hipGetLastError();
}

hipError_t launch_qk_rope(const RopeArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_qk_rope, dim3(a.M, (a.H + 2 * a.KV + 3) / 4), dim3(256), 0, st, QD_ROPE_PRELOAD_ARGS(a), a);
  return hipGetLastError();
}

// 8 waves only where the wave-merge buffers stay small (G * D <= 512); other shapes are
// never instantiated with 8
template <int D, int G, int NW>
static void attn_dec_launch(const AttnDecArgs& a, dim3 grid, hipStream_t st) {
  constexpr int W = (NW == 8 && G * D > 512) ? 4 : NW;
  // the leading (preloaded) arguments: see k_attn_dec
  if (a.nsplit > 8 && a.merge_last == 1)
    hipLaunchKernelGGL((k_attn_dec<D, G, W, true>), grid, dim3(64 * W), 0, st, a.row_slot, a.pos, a.qkv,
                       a.kcache, a.vcache, a.ldqkv, a.KV, a.max_ctx, a.split_len, a);
  else
    hipLaunchKernelGGL((k_attn_dec<D, G, W, false>), grid, dim3(64 * W), 0, st, a.row_slot, a.pos, a.qkv,
                       a.kcache, a.vcache, a.ldqkv, a.KV, a.max_ctx, a.split_len, a);
}

template <int D, int NW>
static hipError_t attn_dec_dw(const AttnDecArgs& a, int G, hipStream_t st) {
  dim3 grid(a.nsplit, a.KV, a.B);
  switch (G) {
    case 1: attn_dec_launch<D, 1, NW>(a, grid, st); break;
    case 2: attn_dec_launch<D, 2, NW>(a, grid, st); break;
    case 3: attn_dec_launch<D, 3, NW>(a, grid, st); break;
    case 4: attn_dec_launch<D, 4, NW>(a, grid, st); break;
    case 5: attn_dec_launch<D, 5, NW>(a, grid, st); break;
    case 6: attn_dec_launch<D, 6, NW>(a, grid, st); break;
    case 7: attn_dec_launch<D, 7, NW>(a, grid, st); break;
    default: attn_dec_launch<D, 8, NW>(a, grid, st); break;
  }
  return hipGetLastError();
}

// 8 waves (128 positions per iteration) when the wave-merge buffers stay small
template <int D>
static hipError_t attn_dec_d(const AttnDecArgs& a, int G, hipStream_t st) {
  if (a.nwaves >= 8 && G * D <= 512) return attn_dec_dw<D, 8>(a, G, st);
  return attn_dec_dw<D, 4>(a, G, st);
}

// the kernel instance launch_attention_decode picks at one split count of eight or fewer
template <int D, int G, int NW>
static const void* attn_dec_kernel() {
  constexpr int W = (NW == 8 && G * D > 512) ? 4 : NW;
  return reinterpret_cast<const void*>(&k_attn_dec<D, G, W, false>);
}
template <int D, int NW>
static const void* attn_dec_kernel_g(int G) {
  switch (G) {
    case 1: return attn_dec_kernel<D, 1, NW>();
    case 2: return attn_dec_kernel<D, 2, NW>();
    case 3: return attn_dec_kernel<D, 3, NW>();
    case 4: return attn_dec_kernel<D, 4, NW>();
    case 5: return attn_dec_kernel<D, 5, NW>();
    case 6: return attn_dec_kernel<D, 6, NW>();
    case 7: return attn_dec_kernel<D, 7, NW>();
    default: return attn_dec_kernel<D, 8, NW>();
  }
}

hipError_t attention_decode_residency(int D, int G, int nwaves, int* blocks) {
  *blocks = 0;
  if (G < 1 || G > 8) return hipErrorInvalidValue;
  const bool w8 = nwaves >= 8 && G * D <= 512;
  const void* k = nullptr;
  switch (D) {
    case 32: k = w8 ? attn_dec_kernel_g<32, 8>(G) : attn_dec_kernel_g<32, 4>(G); break;
    case 64: k = w8 ? attn_dec_kernel_g<64, 8>(G) : attn_dec_kernel_g<64, 4>(G); break;
    case 128: k = w8 ? attn_dec_kernel_g<128, 8>(G) : attn_dec_kernel_g<128, 4>(G); break;
    case 256: k = w8 ? attn_dec_kernel_g<256, 8>(G) : attn_dec_kernel_g<256, 4>(G); break;
    default: return hipErrorInvalidValue;
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, 64 * (w8 ? 8 : 4), 0);
}

hipError_t launch_attention_decode(const AttnDecArgs& a, hipStream_t st) {
  const int G = a.H / a.KV;
  if (G < 1 || G > 8 || a.nsplit < 1) return hipErrorInvalidValue;
  hipError_t e;
  switch (a.D) {
    case 32: e = attn_dec_d<32>(a, G, st); break;
    case 64: e = attn_dec_d<64>(a, G, st); break;
    case 128: e = attn_dec_d<128>(a, G, st); break;
    case 256: e = attn_dec_d<256>(a, G, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.nsplit == 1 || a.merge_last) return e;
  hipLaunchKernelGGL(k_attn_dec_merge, dim3(a.H, a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_flash_prefill(const FlashArgs& a, int n_tiles, int tile_rows, hipStream_t st) {
  if (n_tiles < 1) return hipSuccess;
  if (n_tiles > 65535 || (tile_rows != FLASH_ROWS && tile_rows != 2 * FLASH_ROWS) ||
      (tile_rows == 2 * FLASH_ROWS && a.D > 128))
    return hipErrorInvalidValue;
  dim3 grid(a.H, n_tiles);
  const bool rg2 = tile_rows == 2 * FLASH_ROWS;
  switch (a.D) {
    case 32:
      if (rg2) hipLaunchKernelGGL((k_flash_prefill<32, 2>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a);
      else hipLaunchKernelGGL((k_flash_prefill<32, 1>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a);
      break;
    case 64:
      if (rg2) hipLaunchKernelGGL((k_flash_prefill<64, 2>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a);
      else hipLaunchKernelGGL((k_flash_prefill<64, 1>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a);
      break;
    case 128:
      if (rg2) hipLaunchKernelGGL((k_flash_prefill<128, 2>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a);
      else hipLaunchKernelGGL((k_flash_prefill<128, 1>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a);
      break;
    case 256: hipLaunchKernelGGL((k_flash_prefill<256, 1>), grid, dim3(256), 0, st, QD_FLASH_PRELOAD_ARGS(a), a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


}  // namespace qd
