// Single-sequence (B = 1) decode as one persistent cooperative launch, for gfx950.
//
// The step is the decoder of "Model-agnostic LLM inference", section "Supported models",
// on the int8 weights of section "The quantized load cache" (one fp32 scale per output
// row); the rounding points are those of the multi-kernel path: bf16 after the embedding,
// every RMSNorm, projection, QK-norm, RoPE, attention output, residual sum and
// SiLU(gate) * up; fp32 logits; fp32 accumulation.
//
// One work-group per CU stays resident for all steps of a call.  A layer is five phases --
// q|k|v projection, attention, output projection + residual, gate/up + SiLU, down +
// residual -- and a step ends with the LM head and its arg-max.  Phases are separated by a
// grid barrier (per-XCD arrival counters, XCD leaders on one global counter, one release
// word).  What a phase hands to the next goes through agent-coherent (sc1) stores and
// loads; each wave that stored waits for its stores to complete before the work-group
// arrives, so no L2 write-back or invalidate is needed.
//
// The eight waves have two roles.  Four staging waves load the phase input (written by
// other XCDs), normalize it into LDS, apply the epilogue and run the barrier.  Four weight
// waves hold int8 codes (or K/V tiles) in registers and form the dot products; as soon as
// they are done they request the next phase's codes, so HBM latency overlaps the epilogue
// and the barrier.  The split matters because a wave's memory counter retires loads in
// order: a wave that waited on its activations would also wait on every weight load it
// had issued before them.
//
// Every barrier wait is bounded: a wait that gives up raises an abort word that all
// work-groups poll, and the launch drains with an error flag set.
#include "qd_device.h"

namespace qd {

namespace {

constexpr int PW = PERSIST_WAVES;
constexpr int PT = 64 * PW;
constexpr int NS = PERSIST_SWAVES;   // staging waves 0 .. NS-1
constexpr int NWV = PERSIST_WWAVES;  // weight waves NS .. PW-1
constexpr int PTS = 64 * NS;         // staging threads
constexpr int UMAX = 12;  // weight units (one uint4 per lane) a weight wave holds in registers
constexpr int KSTEP = PERSIST_KSTEP;
constexpr int SC1 = 16;   // buffer cache-policy bit: coherent across the agent's XCDs
constexpr int RSRC_FLAGS = 0x00020000;

// barrier words, each on its own 256-byte line
constexpr int BW_GLOBAL = 0;      // XCD leaders arrive here
constexpr int BW_XCC = 64;        // + 64 * xcc: arrivals of that XCD's work-groups
constexpr int BW_REL = 64 * 17;   // release epoch
constexpr int BW_ABORT = 64 * 18;
constexpr int BW_INIT = 64 * 19;  // start-up rendezvous
constexpr int BW_XCNT = 64 * 20;  // [16] work-groups per XCD

// ---- agent-coherent buffer access ----------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_FLAGS);
}
__device__ __forceinline__ uint4 ld128c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ unsigned long long ld64c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, SC1);
  return ((unsigned long long)v[1] << 32) | v[0];
}
__device__ __forceinline__ uint32_t ld32c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1);
}
__device__ __forceinline__ uint16_t ld16c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, SC1);
}
__device__ __forceinline__ void st16c(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, SC1);
}
__device__ __forceinline__ void st32c(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, SC1);
}
__device__ __forceinline__ void st64c(__amdgpu_buffer_rsrc_t r, uint32_t off, unsigned long long v) {
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  const v2u w = {(unsigned)v, (unsigned)(v >> 32)};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, SC1);
}

__device__ __forceinline__ unsigned ld_ag(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// tensor of layer l at byte offset off from the layer's start (layers repeat at a stride)
template <class T>
__device__ __forceinline__ const T* lwp(const PersistArgs& a, int l, int off) {
  return reinterpret_cast<const T*>(a.lw + (long long)l * a.lstride + off);
}
__device__ __forceinline__ bf16_t* kv_layer(const PersistArgs& a, int l, int which) {
  return a.kv + (long long)(2 * l + which) * a.kvstride;
}

// ---- grid barrier ----------------------------------------------------------------------------
struct Sync {
  unsigned* bar;
  unsigned xcc, members, nx, epoch, lim;
};

// start-up: count the work-groups of each XCD, then meet once on a single counter
__device__ __forceinline__ bool sync_init(Sync& s, unsigned* bar, unsigned lim, int* flag) {
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  s.xcc = xcc & 0xfu;
  s.bar = bar;
  s.epoch = 0;
  s.lim = lim;
  if (threadIdx.x == 0) {
    *flag = 0;
    __hip_atomic_fetch_add(bar + BW_XCNT + s.xcc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(bar + BW_INIT, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(bar + BW_INIT, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < gridDim.x) {
      if (++spins > lim) {
        st_ag(bar + BW_ABORT, 1u);
        *flag = 1;
        break;
      }
    }
  }
  __syncthreads();
  if (*flag) return false;
  s.members = ld_ag(bar + BW_XCNT + s.xcc);
  s.nx = 0;
  for (int i = 0; i < 16; ++i) s.nx += ld_ag(bar + BW_XCNT + i) != 0u ? 1u : 0u;
  return true;
}

// every thread: the staging waves' agent-coherent stores are complete (s_waitcnt 0 in
// each staging wave; the weight waves store nothing that crosses work-groups and keep
// their prefetches in flight), then thread 0 arrives
__device__ __forceinline__ void sync_arrive(Sync& s) {
  if ((threadIdx.x >> 6) < NS) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  s.epoch += 1;
  if (threadIdx.x == 0) {
    const unsigned t = __hip_atomic_fetch_add(s.bar + BW_XCC + 64 * s.xcc, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (t == s.epoch * s.members - 1u) {
      const unsigned g = __hip_atomic_fetch_add(s.bar + BW_GLOBAL, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      if (g == s.epoch * s.nx - 1u) st_ag(s.bar + BW_REL, s.epoch);
    }
  }
}

// thread 0 polls the release word (bounded); false when the launch is being abandoned
__device__ __forceinline__ bool sync_wait(Sync& s, int* flag) {
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (ld_ag(s.bar + BW_REL) < s.epoch) {
      if ((++spins & 255u) == 0u && (spins > s.lim || ld_ag(s.bar + BW_ABORT) != 0u)) {
        st_ag(s.bar + BW_ABORT, 1u);
        *flag = 1;
        break;
      }
    }
  }
  __syncthreads();
  return *flag == 0;
}

// ---- reductions over the staging waves (every wave calls them: they hold block barriers) ----
__device__ __forceinline__ float stage_sum(float v, float* red, int tid) {
  const int lane = tid & 63, wid = tid >> 6;
  if (wid < NS) {
    v = wave_sum(v);
    if (lane == 0) red[wid] = v;
  }
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < NS; ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const unsigned long long t = ((unsigned long long)hi << 32) | lo;
    v = t > v ? t : v;
  }
  return v;
}

__device__ __forceinline__ unsigned long long stage_max_key(unsigned long long v,
                                                            unsigned long long* rkey, int tid) {
  const int lane = tid & 63, wid = tid >> 6;
  if (wid < NS) {
    v = wave_max_key(v);
    if (lane == 0) rkey[wid] = v;
  }
  __syncthreads();
  unsigned long long t = 0ull;
#pragma unroll
  for (int w = 0; w < NS; ++w) t = rkey[w] > t ? rkey[w] : t;
  __syncthreads();
  return t;
}

// ---- one phase's slice of a weight matrix ------------------------------------------------
// A unit is 64 lanes x 16 codes of one row (row r, k-step s); a work-group owns whole rows
// (or whole gate/up pairs) and weight wave v takes units u = v, v + NWV, ...
struct Mat {
  __amdgpu_buffer_rsrc_t rw;  // the whole matrix: loads past its end return zero
  int K, ks, row0, nrows, np, nunits;  // np > 0: nrows = 2 np rows of gate/up pairs
  uint32_t kinv;              // ceil(2^32 / ks) for ks > 1: u / ks = umulhi(u, kinv)
};

// row of unit u (u < 2^16, ks <= 16: the multiply-high quotient is exact)
__device__ __forceinline__ int unit_row(const Mat& m, int u) {
  return m.ks == 1 ? u : (int)__umulhi((uint32_t)u, m.kinv);
}

__device__ __forceinline__ Mat mat_rows(const int8_t* W, int N, int K, int per, int w) {
  Mat m;
  m.rw = rsrc(W, (uint32_t)N * (uint32_t)K);
  m.K = K;
  m.ks = persist_ks(K);
  m.row0 = w * per;
  m.nrows = min(max(N - m.row0, 0), per);
  m.np = 0;
  m.nunits = m.nrows * m.ks;
  m.kinv = m.ks > 1 ? 0xFFFFFFFFu / (uint32_t)m.ks + 1u : 0u;
  return m;
}

// gate/up pairs j0 .. j0 + np - 1: local rows [0, np) are their gate rows, [np, 2 np) the up rows
__device__ __forceinline__ Mat mat_pairs(const int8_t* W, int I, int K, int per, int w) {
  Mat m;
  m.rw = rsrc(W, 2u * (uint32_t)I * (uint32_t)K);
  m.K = K;
  m.ks = persist_ks(K);
  m.row0 = w * per;
  m.np = min(max(I - m.row0, 0), per);
  m.nrows = 2 * m.np;
  m.nunits = m.nrows * m.ks;
  m.kinv = m.ks > 1 ? 0xFFFFFFFFu / (uint32_t)m.ks + 1u : 0u;
  return m;
}

__device__ __forceinline__ int mat_row(const Mat& m, int lr) {
  if (m.np > 0) return lr < m.np ? gu_row(m.row0 + lr, 0) : gu_row(m.row0 + lr - m.np, 1);
  return m.row0 + lr;
}

constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer: the load returns zero

// branch-free: a unit past the slice, or lanes past the end of the row, read zeros
__device__ __forceinline__ uint4 mat_load(const Mat& m, int u, int lane) {
  const int lr = unit_row(m, u), s = u - lr * m.ks, c = s * KSTEP + 16 * lane;
  const uint32_t raw = (uint32_t)mat_row(m, lr) * (uint32_t)m.K + (uint32_t)c;
  const uint32_t off = (u < m.nunits && c < m.K) ? raw : OOB;
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(m.rw, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void mat_prefetch(const Mat& m, uint4 (&wb)[UMAX], int wv, int lane) {
#pragma unroll
  for (int i = 0; i < UMAX; ++i) wb[i] = mat_load(m, wv + NWV * i, lane);
}

// wave dot product of unit u with the staged input xs (bf16 in LDS); lanes past the end
// of the row hold zero codes and read an in-range slice of xs
__device__ __forceinline__ float unit_dot(const Mat& m, int u, const uint4 w, const bf16_t* xs,
                                          int lane) {
  const int lr = unit_row(m, u), s = u - lr * m.ks, c = s * KSTEP + 16 * lane;
  const uint4* xp = reinterpret_cast<const uint4*>(xs + (c < m.K ? c : 0));
  const uint4 x0 = xp[0], x1 = xp[1];
  float wf[16];
  i8x16_to_f32(make_int4((int)w.x, (int)w.y, (int)w.z, (int)w.w), wf);
  const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc = fmaf(wf[2 * j], __uint_as_float(xw[j] << 16), acc);
    acc = fmaf(wf[2 * j + 1], __uint_as_float(xw[j] & 0xFFFF0000u), acc);
  }
  return wave_sum(c < m.K ? acc : 0.0f);
}

// all units of the slice on one weight wave: the first UMAX come from wb (already
// requested); the rest stream through in chunks, each requested before the previous one
// is used.  Unit results go to part[u] in LDS.
__device__ __forceinline__ void mat_run(const Mat& m, uint4 (&wb)[UMAX], const bf16_t* xs,
                                        float* part, int wv, int lane) {
  constexpr int PER = NWV * UMAX;
  for (int base = 0; base < m.nunits; base += PER) {
    const bool more = base + PER < m.nunits;
    uint4 nx[UMAX];
    if (more) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i) nx[i] = mat_load(m, base + PER + wv + NWV * i, lane);
    }
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      const int u = base + wv + NWV * i;
      if (u < m.nunits) {
        const float v = unit_dot(m, u, wb[i], xs, lane);
        if (lane == 0) part[u] = v;
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i) wb[i] = nx[i];
    }
  }
}

__device__ __forceinline__ float row_acc(const Mat& m, const float* part, int lr) {
  float a = 0.0f;
  for (int s = 0; s < m.ks; ++s) a += part[lr * m.ks + s];
  return a;
}

// ---- phase inputs staged in LDS by the staging waves (every wave calls these) ------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// RMSNorm of a K-vector (K <= PERSIST_MAX_D) into xs: y = bf16(x / sqrt(mean(x^2) + eps) *
// gain).  x is the residual stream (agent-coherent loads from g) or, with erow set, the
// embedding row x = bf16(code * escale); then the raw rows [own0, own0 + nown) also go to
// xown.
__device__ __forceinline__ void stage_norm(const bf16_t* g, const int8_t* erow, float escale,
                                           int K, const float* gain, float eps, bf16_t* xs,
                                           float* red, bf16_t* xown, int own0, int nown, int tid) {
  const int nch = K >> 3;
  const bool act = tid < PTS;
  const __amdgpu_buffer_rsrc_t rg = rsrc(g, (uint32_t)K * 2u);
  uint4 xr[4];
  float4 g0[4], g1[4];
  float ss = 0.0f;
  if (act) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + PTS * i;
      xr[i] = make_uint4(0u, 0u, 0u, 0u);
      g0[i] = g1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nch) {
        if (erow) {
          const uint2 q = *reinterpret_cast<const uint2*>(erow + 8 * c);
          const uint32_t qb[2] = {q.x, q.y};
          uint32_t wv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t word = qb[j >> 1];
            const int e0 = 2 * (j & 1), e1 = e0 + 1;
            const float f0 = (float)((int)(word << (24 - 8 * e0)) >> 24) * escale;
            const float f1 = (float)((int)(word << (24 - 8 * e1)) >> 24) * escale;
            wv[j] = (uint32_t)f2bf(f0) | ((uint32_t)f2bf(f1) << 16);
          }
          xr[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        } else {
          xr[i] = ld128c(rg, 16u * (uint32_t)c);
        }
        const float4* gp = reinterpret_cast<const float4*>(gain + 8 * c);
        g0[i] = gp[0];
        g1[i] = gp[1];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w4[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = bf_lo(w4[j]), b = bf_hi(w4[j]);
        ss += a * a + b * b;
      }
    }
  }
  const float rinv = 1.0f / sqrtf(stage_sum(ss, red, tid) / (float)K + eps);
  if (act) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + PTS * i;
      if (c < nch) {
        const uint32_t w4[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        const float gv[8] = {g0[i].x, g0[i].y, g0[i].z, g0[i].w, g1[i].x, g1[i].y, g1[i].z, g1[i].w};
        uint32_t o4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16_t y0 = f2bf(bf_lo(w4[j]) * rinv * gv[2 * j]);
          const bf16_t y1 = f2bf(bf_hi(w4[j]) * rinv * gv[2 * j + 1]);
          o4[j] = (uint32_t)y0 | ((uint32_t)y1 << 16);
        }
        *reinterpret_cast<uint4*>(xs + 8 * c) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
        if (xown) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * c + e - own0;
            if (r >= 0 && r < nown) xown[r] = (bf16_t)(w4[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  }
  __syncthreads();
}

// plain copy of a K-vector (agent-coherent loads, four chunks per thread in flight) into xs
__device__ __forceinline__ void stage_copy(const bf16_t* g, int K, bf16_t* xs, int tid) {
  const int nch = K >> 3;
  if (tid < PTS) {
    const __amdgpu_buffer_rsrc_t rg = rsrc(g, (uint32_t)K * 2u);
    for (int c0 = tid; c0 < nch; c0 += 4 * PTS) {
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + PTS * i;
        v[i] = ld128c(rg, c < nch ? 16u * (uint32_t)c : OOB);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + PTS * i;
        if (c < nch) *reinterpret_cast<uint4*>(xs + 8 * c) = v[i];
      }
    }
  }
  __syncthreads();
}

// attention output of every head from the split partials (agent-coherent loads):
// o = sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M), rounded to bf16, into xs [H*D].
// The partials of a thread's first four outputs (splits 0..3) are requested together with
// the (max, sum) pairs, so the common case is one memory round trip.
__device__ __forceinline__ void stage_merge(const float* po, const float* pml, int H, int D,
                                            int nsplit, bf16_t* xs, float* mf, int tid) {
  const bool act = tid < PTS;
  const __amdgpu_buffer_rsrc_t rml = rsrc(pml, (uint32_t)H * PERSIST_SPLITS * 8u);
  const __amdgpu_buffer_rsrc_t rpo = rsrc(po, (uint32_t)H * PERSIST_SPLITS * D * 4u);
  const int HDv = H * D, e0 = 4 * tid;
  const int h0 = e0 < HDv ? e0 / D : 0, dd0 = e0 - h0 * D;
  uint4 v0[4];
  if (act) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v0[k] = ld128c(rpo, (e0 < HDv && k < nsplit)
                              ? 4u * (uint32_t)((h0 * PERSIST_SPLITS + k) * D + dd0)
                              : OOB);
    for (int i = tid; i < H * nsplit; i += PTS) {
      const int h = i / nsplit, s = i - h * nsplit;
      const int pi = h * PERSIST_SPLITS + s;
      const unsigned long long v = ld64c(rml, 8u * (uint32_t)pi);
      mf[2 * pi] = __uint_as_float((uint32_t)v);
      mf[2 * pi + 1] = __uint_as_float((uint32_t)(v >> 32));
    }
  }
  __syncthreads();
  float* Lh = mf + 2 * H * PERSIST_SPLITS;
  if (act) {
    for (int h = tid; h < H; h += PTS) {
      float M = -INFINITY;
      for (int s = 0; s < nsplit; ++s) M = fmaxf(M, mf[2 * (h * PERSIST_SPLITS + s)]);
      float L = 0.0f;
      for (int s = 0; s < nsplit; ++s) {
        const int pi = h * PERSIST_SPLITS + s;
        const float ms = mf[2 * pi];
        const float f = ms == -INFINITY ? 0.0f : expf(ms - M);
        L += mf[2 * pi + 1] * f;
        mf[2 * pi] = f;  // the weight of split s replaces its max
      }
      Lh[h] = L;
    }
  }
  __syncthreads();
  if (act) {
    for (int e = e0; e < HDv; e += 4 * PTS) {
      const int h = e / D, dd = e - h * D;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < nsplit; s0 += 4) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v[k] = (e == e0 && s0 == 0)
                     ? v0[k]
                     : ld128c(rpo, s0 + k < nsplit
                                       ? 4u * (uint32_t)((h * PERSIST_SPLITS + s0 + k) * D + dd)
                                       : OOB);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (s0 + k < nsplit) {
            const float f = mf[2 * (h * PERSIST_SPLITS + s0 + k)];
            acc[0] += __uint_as_float(v[k].x) * f;
            acc[1] += __uint_as_float(v[k].y) * f;
            acc[2] += __uint_as_float(v[k].z) * f;
            acc[3] += __uint_as_float(v[k].w) * f;
          }
        }
      }
      const float L = Lh[h];
      const uint32_t lo = (uint32_t)f2bf(acc[0] / L) | ((uint32_t)f2bf(acc[1] / L) << 16);
      const uint32_t hi = (uint32_t)f2bf(acc[2] / L) | ((uint32_t)f2bf(acc[3] / L) << 16);
      *reinterpret_cast<uint2*>(xs + e) = make_uint2(lo, hi);
    }
  }
  __syncthreads();
}

// ---- attention of one (KV head, position split) --------------------------------------------
template <int D>
struct Att {
  static constexpr int HALF = D / 2;
  static constexpr int KQ = D / 4;                   // key elements per lane (4 lanes a position)
  static constexpr int KV4 = KQ / 8;                 // uint4 loads per lane per key row
  static constexpr int DPL = D >= 64 ? D / 64 : 1;   // value dims per lane
  static constexpr int VW = DPL >= 2 ? DPL / 2 : 1;  // 32-bit words of V per lane per position
};

// K/V tiles of one iteration for weight wave v: lane (tl = lane / 4, part = lane % 4) holds
// key elements [part*KQ, part*KQ + KQ) of position t0 + 16 v + tl, and the values of the
// wave's 16 positions for its own dims.  Position p (written in this phase) reads as zero.
template <int D>
__device__ __forceinline__ void attn_tiles(uint4 (&kk)[Att<D>::KV4], uint32_t (&vv)[16][Att<D>::VW],
                                           __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           int t0, int te, int p, int wv, int lane) {
  using C = Att<D>;
  const int tl = lane >> 2, part = lane & 3;
  const int t = t0 + 16 * wv + tl;
  const bool vlane = (D >= 64) || (lane < D);
  const bool kok = t < te && t != p;
#pragma unroll
  for (int j = 0; j < C::KV4; ++j)
    kk[j] = ld128c(rk, kok ? 2u * (uint32_t)(t * D + part * C::KQ + 8 * j) : OOB);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tv = t0 + 16 * wv + i;
    const bool ok = tv < te && tv != p && vlane;
#pragma unroll
    for (int w = 0; w < C::VW; ++w) {
      if (C::DPL >= 2)
        vv[i][w] = ld32c(rv, ok ? 2u * (uint32_t)(tv * D + C::DPL * lane + 2 * w) : OOB);
      else
        vv[i][w] = (uint32_t)ld16c(rv, ok ? 2u * (uint32_t)(tv * D + lane) : OOB);
    }
  }
}

// Staging waves: QK-norm and RoPE of the group's G query heads and its key head at
// position p (from the raw projections); the split holding p writes K/V row p.  Weight
// waves: online softmax over their positions with the tiles already in registers.  Then the
// staging threads merge the weight waves and publish the split's partials per head.
template <int D, int GM>
__device__ __forceinline__ void attn_item(const PersistArgs& a, int layer, int g, int s,
                                          int split_len, int p, float* att,
                                          uint4 (&kc)[Att<D>::KV4],
                                          uint32_t (&vc)[16][Att<D>::VW], int tid) {
  using C = Att<D>;
  const int wid = tid >> 6, lane = tid & 63;
  const int G = a.H / a.KV, n = p + 1;
  const int tb = s * split_len, te = min(n, tb + split_len);
  const int tl = lane >> 2, part = lane & 3;
  float* qs = att;              // [G][D]
  float* kn = qs + G * D;       // [D]
  float* vn = kn + D;           // [D]
  float* wm = vn + D;           // [NWV][G]
  float* wl = wm + NWV * G;     // [NWV][G]
  float* wo = wl + NWV * G;     // [NWV][G][D]
  const bool owner = tb <= p && p < tb + split_len;
  const bool vlane = (D >= 64) || (lane < D);
  const int HD = a.H * D, KVD = a.KV * D;
  const uint32_t kvbytes = (uint32_t)a.max_ctx * D * 2u;
  const __amdgpu_buffer_rsrc_t rk = rsrc(kv_layer(a, layer, 0) + (size_t)g * a.max_ctx * D, kvbytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(kv_layer(a, layer, 1) + (size_t)g * a.max_ctx * D, kvbytes);

  if (wid < NS) {
    const __amdgpu_buffer_rsrc_t rq = rsrc(a.qkvg, (uint32_t)(HD + 2 * KVD) * 2u);
    const float2* tab = a.rope + (size_t)p * C::HALF;
    for (int hh = wid; hh <= G; hh += NS) {
      const bool isq = hh < G;
      const int base = isq ? (g * G + hh) * D : HD + g * D;
      const float* gn = lwp<float>(a, layer, isq ? a.lo.qn_g : a.lo.kn_g);
      float x1[2], x2[2], ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = lane + 64 * j;
        x1[j] = x2[j] = 0.0f;
        if (i < C::HALF) {
          x1[j] = bf2f(ld16c(rq, 2u * (uint32_t)(base + i)));
          x2[j] = bf2f(ld16c(rq, 2u * (uint32_t)(base + i + C::HALF)));
          ss += x1[j] * x1[j] + x2[j] * x2[j];
        }
      }
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = lane + 64 * j;
        if (i < C::HALF) {
          const float y1 = rbf(x1[j] * inv * gn[i]);
          const float y2 = rbf(x2[j] * inv * gn[i + C::HALF]);
          const float2 cs = tab[i];
          const bf16_t o1 = f2bf(y1 * cs.x - y2 * cs.y), o2 = f2bf(y2 * cs.x + y1 * cs.y);
          if (isq) {
            qs[hh * D + i] = bf2f(o1);
            qs[hh * D + i + C::HALF] = bf2f(o2);
          } else {
            kn[i] = bf2f(o1);
            kn[i + C::HALF] = bf2f(o2);
            if (owner) {
              st16c(rk, 2u * (uint32_t)(p * D + i), o1);
              st16c(rk, 2u * (uint32_t)(p * D + i + C::HALF), o2);
            }
          }
        }
      }
    }
    for (int i = tid; i < D; i += PTS) {
      const bf16_t v = ld16c(rq, 2u * (uint32_t)(HD + KVD + g * D + i));
      vn[i] = bf2f(v);
      if (owner) st16c(rv, 2u * (uint32_t)(p * D + i), v);
    }
  }
  __syncthreads();

  if (wid >= NS) {
    const int wv = wid - NS;
    const float scale = 1.0f / sqrtf((float)D);
    float m[GM], l[GM], o[GM][C::DPL];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < C::DPL; ++e) o[h][e] = 0.0f;
    }
    for (int t0 = tb; t0 < te; t0 += PERSIST_CHUNK) {
      const int t = t0 + 16 * wv + tl;
      float sp[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) sp[h] = 0.0f;
      if (t == p) {
        for (int j = 0; j < C::KQ; ++j) {
          const float kv = kn[part * C::KQ + j];
#pragma unroll
          for (int h = 0; h < GM; ++h)
            if (h < G) sp[h] += qs[h * D + part * C::KQ + j] * kv;
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::KV4; ++j) {
          const uint32_t w4[4] = {kc[j].x, kc[j].y, kc[j].z, kc[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float k0 = bf_lo(w4[e]), k1 = bf_hi(w4[e]);
            const int c = part * C::KQ + 8 * j + 2 * e;
#pragma unroll
            for (int h = 0; h < GM; ++h)
              if (h < G) sp[h] += qs[h * D + c] * k0 + qs[h * D + c + 1] * k1;
          }
        }
      }
      const bool more = t0 + PERSIST_CHUNK < te;
      uint4 kx[C::KV4];
      uint32_t vx[16][C::VW];
      if (more) attn_tiles<D>(kx, vx, rk, rv, t0 + PERSIST_CHUNK, te, p, wv, lane);
      const bool valid = t < te;
      float pr[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        pr[h] = 0.0f;
        if (h < G) {
          sp[h] += __shfl_xor(sp[h], 1, 64);
          sp[h] += __shfl_xor(sp[h], 2, 64);
          const float z = valid ? sp[h] * scale : -INFINITY;
          const float mnew = fmaxf(m[h], wave_max(z));
          const float alpha = (m[h] == -INFINITY) ? 0.0f : expf(m[h] - mnew);
          pr[h] = valid ? expf(z - mnew) : 0.0f;
          l[h] = l[h] * alpha + wave_sum(part == 0 ? pr[h] : 0.0f);
          m[h] = mnew;
#pragma unroll
          for (int e = 0; e < C::DPL; ++e) o[h][e] *= alpha;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tv = t0 + 16 * wv + i;
        float vf[C::DPL];
        if (tv == p) {
#pragma unroll
          for (int e = 0; e < C::DPL; ++e) vf[e] = vlane ? vn[C::DPL * lane + e] : 0.0f;
        } else if (C::DPL >= 2) {
#pragma unroll
          for (int w = 0; w < C::VW; ++w) {
            vf[2 * w] = bf_lo(vc[i][w]);
            vf[2 * w + 1] = bf_hi(vc[i][w]);
          }
        } else {
          vf[0] = bf_lo(vc[i][0]);
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h < G) {
            const float pw = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[h]), 4 * i));
#pragma unroll
            for (int e = 0; e < C::DPL; ++e) o[h][e] += pw * vf[e];
          }
        }
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < C::KV4; ++j) kc[j] = kx[j];
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int w = 0; w < C::VW; ++w) vc[i][w] = vx[i][w];
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        if (lane == 0) {
          wm[wv * G + h] = m[h];
          wl[wv * G + h] = l[h];
        }
        if (vlane) {
#pragma unroll
          for (int e = 0; e < C::DPL; ++e) wo[(wv * G + h) * D + C::DPL * lane + e] = o[h][e];
        }
      }
    }
  }
  __syncthreads();
  if (wid < NS) {
    const __amdgpu_buffer_rsrc_t rpo = rsrc(a.po, (uint32_t)a.H * PERSIST_SPLITS * D * 4u);
    const __amdgpu_buffer_rsrc_t rml = rsrc(a.pml, (uint32_t)a.H * PERSIST_SPLITS * 8u);
    for (int idx = tid; idx < G * D; idx += PTS) {
      const int h = idx / D, dd = idx - h * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWV; ++w) M = fmaxf(M, wm[w * G + h]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        if (wm[w * G + h] == -INFINITY) continue;
        const float f = expf(wm[w * G + h] - M);
        L += wl[w * G + h] * f;
        O += wo[(w * G + h) * D + dd] * f;
      }
      const int pi = (g * G + h) * PERSIST_SPLITS + s;
      st32c(rpo, 4u * (uint32_t)(pi * D + dd), __float_as_uint(O));
      if (dd == 0) {
        st32c(rml, 8u * (uint32_t)pi, __float_as_uint(M));
        st32c(rml, 8u * (uint32_t)pi + 4u, __float_as_uint(L));
      }
    }
  }
}

// ---- the kernel ------------------------------------------------------------------------------
// Phases of a step are numbered ph = 5 l + t (t: 0 q|k|v, 1 attention, 2 output projection,
// 3 gate/up, 4 down) and ph = 5 L is the LM head.  One copy of each phase body serves every
// layer, so the per-phase values are computed where they are used.
struct Dims {
  int d, H, KV, D, I, V, HD, KVD, NQKV, rq, rd, rp, rv;
};

__device__ __forceinline__ Mat phase_mat(const PersistArgs& a, const Dims& z, int ph, int w) {
  if (ph >= 5 * a.L) return mat_rows(a.emb_q, z.V, z.d, z.rv, w);
  const int l = ph / 5, t = ph - 5 * l;
  if (t == 3) return mat_pairs(lwp<int8_t>(a, l, a.lo.gu_q), z.I, z.d, z.rp, w);
  const int8_t* W = lwp<int8_t>(a, l, t == 0 ? a.lo.qkv_q : (t == 2 ? a.lo.o_q : a.lo.dn_q));
  const int N = t == 0 ? z.NQKV : z.d;
  const int K = t == 0 ? z.d : (t == 2 ? z.HD : z.I);
  return mat_rows(W, N, K, t == 0 ? z.rq : z.rd, w);
}

template <int D, int GM>
__global__ __launch_bounds__(PT) void k_decode_persist(PersistArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  using C = Att<D>;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int w = blockIdx.x, nwg = gridDim.x;
  const PersistLds lay = persist_lds(a.d, a.H, a.KV, D, a.I, a.V, nwg);
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem + lay.xs);
  float* part = reinterpret_cast<float*>(smem + lay.part);
  float* red = reinterpret_cast<float*>(smem + lay.red);
  unsigned long long* rkey = reinterpret_cast<unsigned long long*>(smem + lay.rkey);
  bf16_t* xown = reinterpret_cast<bf16_t*>(smem + lay.xown);
  float* att = reinterpret_cast<float*>(smem + lay.att);
  float* mf = reinterpret_cast<float*>(smem + lay.mf);
  int* flag = reinterpret_cast<int*>(smem + lay.flag);

  Dims z;
  z.d = a.d; z.H = a.H; z.KV = a.KV; z.D = D; z.I = a.I; z.V = a.V;
  z.HD = a.H * D; z.KVD = a.KV * D; z.NQKV = z.HD + 2 * z.KVD;
  z.rq = persist_cdiv(z.NQKV, nwg); z.rd = persist_cdiv(a.d, nwg);
  z.rp = persist_cdiv(a.I, nwg); z.rv = persist_cdiv(a.V, nwg);
  const int own0 = w * z.rd, nown = min(max(a.d - own0, 0), z.rd);
  const int nph = 5 * a.L + 1;

  uint4 wb[UMAX];
  uint4 kc[C::KV4];
  uint32_t vc[16][C::VW];
  Sync S;

  // the first projection's codes go out before the start-up rendezvous
  if (wid >= NS) mat_prefetch(phase_mat(a, z, 0, w), wb, wid - NS, lane);
  if (!sync_init(S, a.bar, a.spin_limit, flag)) {
    if (tid == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int p0 = a.pos[0];
  int id = min(max(a.in_id[0], 0), a.V - 1);

  for (int step = 0; step < a.nsteps; ++step) {
    const int p = p0 + step, n = p + 1;
    // position splits of this step: chunks of PERSIST_CHUNK, at most one work-group each
    const int chunks = persist_cdiv(n, PERSIST_CHUNK);
    const int smax = max(1, min(min(PERSIST_SPLITS, a.max_splits), nwg / a.KV));
    const int split_len = persist_cdiv(chunks, min(chunks, smax)) * PERSIST_CHUNK;
    const int nsplit = persist_cdiv(n, split_len);
    const bool has_item = w < a.KV * nsplit;
    const int ig = has_item ? w / nsplit : 0, is = has_item ? w - ig * nsplit : 0;

    for (int ph = 0; ph < nph; ++ph) {
      // the thread index is re-read opaquely in every phase, so the compiler recomputes
      // the per-thread offsets here instead of keeping them live across the whole launch
      int tq = tid;
      asm volatile("" : "+v"(tq));
      const int lq = tq & 63, wq = tq >> 6;
      const bool sw = wq < NS;  // staging wave
      const int l = ph / 5, t = ph - 5 * l;
      const bool lm = ph == nph - 1;
      if (!lm && t == 1) {
        // ---- attention (weight waves request the output projection's codes first) ----
        if (!sw) mat_prefetch(phase_mat(a, z, ph + 1, w), wb, wq - NS, lq);
        if (has_item) attn_item<D, GM>(a, l, ig, is, split_len, p, att, kc, vc, tq);
      } else {
        // ---- a projection: stage its input in LDS, run the units, apply the epilogue ----
        const Mat m = phase_mat(a, z, ph, w);
        const float* sp =
            lm ? a.emb_s
               : lwp<float>(a, l, t == 0 ? a.lo.qkv_s : (t == 2 ? a.lo.o_s : (t == 3 ? a.lo.gu_s : a.lo.dn_s)));
        // scales of this staging thread's output rows (gate/up: both halves; LM head: up to 4)
        float s0 = 0.0f, s1 = 0.0f, sv[4] = {0.f, 0.f, 0.f, 0.f};
        if (sw) {
          if (lm) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (tq + PTS * k < m.nrows) sv[k] = sp[m.row0 + tq + PTS * k];
          } else if (tq < (t == 3 ? m.np : m.nrows)) {
            s0 = sp[t == 3 ? gu_row(m.row0 + tq, 0) : m.row0 + tq];
            if (t == 3) s1 = sp[gu_row(m.row0 + tq, 1)];
          }
        }
        if (!lm && t == 2) {
          stage_merge(a.po, a.pml, a.H, D, nsplit, xs, mf, tq);
        } else if (!lm && t == 4) {
          stage_copy(a.actg, a.I, xs, tq);
        } else {
          const float* gain = lm ? a.final_g : lwp<float>(a, l, t == 0 ? a.lo.in_g : a.lo.post_g);
          const bool emb = !lm && t == 0 && l == 0;
          stage_norm(a.xg, emb ? a.emb_q + (size_t)id * a.d : nullptr, emb ? a.emb_s[id] : 0.0f,
                     a.d, gain, a.eps, xs, red, emb ? xown : nullptr, own0, nown, tq);
        }
        if (!sw) {
          const int wv = wq - NS;
          mat_run(m, wb, xs, part, wv, lq);
          // the next phase's requests go out now, ahead of the epilogue and the barrier
          if (!lm && t == 0) {
            if (has_item) {
              const uint32_t kvbytes = (uint32_t)a.max_ctx * D * 2u;
              attn_tiles<D>(kc, vc, rsrc(kv_layer(a, l, 0) + (size_t)ig * a.max_ctx * D, kvbytes),
                            rsrc(kv_layer(a, l, 1) + (size_t)ig * a.max_ctx * D, kvbytes),
                            is * split_len, min(n, is * split_len + split_len), p, wv, lq);
            }
          } else if (!lm) {
            mat_prefetch(phase_mat(a, z, ph + 1, w), wb, wv, lq);
          } else if (step + 1 < a.nsteps) {
            mat_prefetch(phase_mat(a, z, 0, w), wb, wv, lq);
          }
        }
        __syncthreads();
        if (lm) {
          const bool want_logits = a.logits != nullptr && step == a.nsteps - 1;
          unsigned long long best = 0ull;
          if (sw) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int r0 = tq + PTS * k;
              if (r0 < m.nrows) {
                const int r = m.row0 + r0;
                const float v = row_acc(m, part, r0) * sv[k];
                if (want_logits) a.logits[r] = v;
                const unsigned long long key = argmax_key(v, r);
                best = key > best ? key : best;
              }
            }
          }
          best = stage_max_key(best, rkey, tq);
          if (tq == 0) st64c(rsrc(a.keys, (uint32_t)nwg * 8u), 8u * (uint32_t)w, best);
        } else if (sw) {
          if (t == 0) {
            if (tq < m.nrows)
              st16c(rsrc(a.qkvg, (uint32_t)z.NQKV * 2u), 2u * (uint32_t)(m.row0 + tq),
                    f2bf(row_acc(m, part, tq) * s0));
          } else if (t == 3) {
            if (tq < m.np) {
              const float gv = rbf(row_acc(m, part, tq) * s0);
              const float uv = rbf(row_acc(m, part, m.np + tq) * s1);
              st16c(rsrc(a.actg, (uint32_t)a.I * 2u), 2u * (uint32_t)(m.row0 + tq),
                    f2bf(gv / (1.0f + expf(-gv)) * uv));
            }
          } else if (tq < m.nrows) {  // t == 2 or 4: residual rows kept by this work-group
            const bf16_t xn = f2bf(bf2f(xown[tq]) + rbf(row_acc(m, part, tq) * s0));
            xown[tq] = xn;
            st16c(rsrc(a.xg, (uint32_t)a.d * 2u), 2u * (uint32_t)(m.row0 + tq), xn);
          }
        }
      }
      sync_arrive(S);
      if (!sync_wait(S, flag)) {
        if (tq == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
    // ---- every work-group reduces the keys to the next id ----
    {
      int tq = tid;
      asm volatile("" : "+v"(tq));
      unsigned long long k = 0ull;
      if (tq < PTS) {
        const __amdgpu_buffer_rsrc_t rkeys = rsrc(a.keys, (uint32_t)nwg * 8u);
        for (int t = tq; t < nwg; t += PTS) {
          const unsigned long long v = ld64c(rkeys, 8u * (uint32_t)t);
          k = v > k ? v : k;
        }
      }
      k = stage_max_key(k, rkey, tq);
      id = min(max(key_index(k), 0), a.V - 1);
      if (w == 0 && tq == 0 && a.out_ids) a.out_ids[step] = id;
    }
  }
  if (w == 0 && tid == 0) {
    a.next_id[0] = id;
    a.pos[0] = p0 + a.nsteps;
  }
}

}  // namespace

namespace {
// kernel instance for head_dim D and G query heads per KV head (G rounded up to 2, 4, 8)
const void* persist_kernel(int D, int G) {
  const int gm = G <= 2 ? 2 : (G <= 4 ? 4 : (G <= 8 ? 8 : 0));
#define QD_K(d, g) if (D == d && gm == g) return reinterpret_cast<const void*>(k_decode_persist<d, g>)
  QD_K(32, 2); QD_K(32, 4); QD_K(32, 8);
  QD_K(64, 2); QD_K(64, 4); QD_K(64, 8);
  QD_K(128, 2); QD_K(128, 4); QD_K(128, 8);
#undef QD_K
  return nullptr;
}
}  // namespace

hipError_t persist_occupancy(int D, int G, int lds, int* blocks) {
  *blocks = 0;
  const void* k = persist_kernel(D, G);
  if (!k) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, PT, lds);
}

hipError_t launch_decode_persistent(const PersistArgs& a, int nwg, int lds, hipStream_t st) {
  const void* k = persist_kernel(a.D, a.H / a.KV);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = launch_fill_i32(reinterpret_cast<int*>(a.bar), PERSIST_BAR_WORDS, 0, st);
  if (e != hipSuccess) return e;
  void* args[] = {const_cast<PersistArgs*>(&a)};
  return hipLaunchCooperativeKernel(k, dim3(nwg), dim3(PT), args, lds, st);
}

}  // namespace qd
