// Sampled decode ("Model-agnostic LLM inference", section "Sampling"): the chain
// repetition / presence / frequency penalties -> temperature -> top-k -> min-p -> top-p
// -> seeded weighted draw, on the device, one work-group per logits row.
//
// Readings (the pages name the steps, not their formulas): counts are the occurrences of
// each token in the sequence so far (prompt and every token fed since, counted by the
// embedding kernel); a seen token's logit is divided by the repetition penalty when
// positive and multiplied by it otherwise, then presence + frequency * count is
// subtracted; the result is divided by the temperature.  Top-k keeps the k largest
// (equal values: lower token id first).  Min-p keeps probabilities >= min_p times the
// largest; top-p the shortest prefix of what is left whose mass reaches top_p of it.  The
// draw takes u in [0, 1) from Philox4x64-10 (Salmon et al., SC 2011) with key (seed, 0)
// and counter (n, 0, 0, 0), n = draws so far for the sequence, u = top 24 bits of the
// first word times 2^-24, and picks the first candidate whose cumulative weight exceeds
// u times the kept weight.
//
// The k-th largest value is found exactly by a radix select over the distance of an
// order-preserving 32-bit key from the row's largest (histograms in LDS); the candidates (every key >= that
// value) are sorted in LDS by (value descending, id ascending); weights, min-p, top-p
// and the draw are block-wide counts over a fixed-order prefix sum.
#include "qd_common.h"
#include "qd_device.h"

#include <map>
#include <mutex>

namespace qd {

namespace {
constexpr int SMP_T = 1024;            // threads of the finishing work-group of a row
constexpr int SMP_CAND = SMP_CAND_G;    // LDS candidate capacity (the gathered list)
constexpr int SMP_CHUNK = 4096;         // row elements per streaming work-group

// order-preserving key: larger value, larger key; -0.0 and +0.0 share a key
__device__ __forceinline__ uint32_t fkey(float v) {
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Philox4x64-10, first output word
__device__ __forceinline__ unsigned long long philox_word0(unsigned long long c0,
                                                           unsigned long long key0) {
  const unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  unsigned long long x0 = c0, x1 = 0, x2 = 0, x3 = 0, k0 = key0, k1 = 0;
  for (int r = 0; r < 10; ++r) {
    const unsigned long long hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    const unsigned long long hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return x0;
}

constexpr int SMP_U = 16;  // elements per thread per loop trip (loads issued together)

// inclusive prefix sum over the block in thread order (fixed order: wave scans, then the
// wave totals)
__device__ __forceinline__ float block_scan(float v, float* wsum) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float run = 0.0f;
    for (int w = 0; w < SMP_T / 64; ++w) {
      const float t = wsum[w];
      wsum[w] = run;
      run += t;
    }
  }
  __syncthreads();
  return v + wsum[wid];
}
}  // namespace

// ---- streaming passes: many work-groups per row -----------------------------------------

// penalized, tempered logits of one chunk into the scratch row; the row's largest key
__global__ __launch_bounds__(256) void k_smp_prep(SampleArgs a) {
  __shared__ uint32_t wmax[4];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sl = a.row_slot ? a.row_slot[b] : b;
  const int V = a.V;
  const float* lg = a.logits + (size_t)b * a.ldl;
  float* zr = a.z + (size_t)b * V;
  const int* cr = a.counts + (size_t)sl * V;
  const int v_end = min(V, (int)(blockIdx.x + 1) * SMP_CHUNK);
  uint32_t kmax = 0u;
  for (int v0 = blockIdx.x * SMP_CHUNK; v0 < v_end; v0 += 4 * 256) {
    float l[4];
    int c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // clamped (valid) indices: every load goes out first
      const int v = v0 + u * 256 + tid;
      l[u] = lg[v < v_end ? v : 0];
      c[u] = cr[v < v_end ? v : 0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 256 + tid;
      float x = l[u];
      if (c[u] > 0) {
        x = x > 0.0f ? x / a.repeat_penalty : x * a.repeat_penalty;
        x -= a.presence_penalty + a.frequency_penalty * (float)c[u];
      }
      const float z = x / a.temperature;
      if (v < v_end) {
        zr[v] = z;
        kmax = max(kmax, fkey(z));
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  if (lane == 0) wmax[wid] = kmax;
  __syncthreads();
  if (tid == 0) atomicMax(a.rowmax + b, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

// histogram of the key distance from the row's largest, d < 2^24, bins of 2^16
__global__ __launch_bounds__(256) void k_smp_hist(SampleArgs a) {
  __shared__ unsigned int h[256];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int V = a.V;
  const float* zr = a.z + (size_t)b * V;
  h[tid] = 0u;
  __syncthreads();
  const uint32_t maxk = a.rowmax[b];
  const int v_end = min(V, (int)(blockIdx.x + 1) * SMP_CHUNK);
  for (int v0 = blockIdx.x * SMP_CHUNK; v0 < v_end; v0 += 4 * 256) {
    float zz[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 256 + tid;
      zz[u] = zr[v < v_end ? v : 0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 256 + tid;
      const uint32_t d = maxk - fkey(zz[u]);
      if (v < v_end && d < (1u << 24)) atomicAdd(&h[d >> 16], 1u);
    }
  }
  __syncthreads();
  if (h[tid]) atomicAdd(a.hist + (size_t)b * 256 + tid, h[tid]);
}

// the bin of the k-th largest (from the histogram), then every element of this chunk at
// that distance or closer into the row's candidate list (one counter update per wave)
__global__ __launch_bounds__(256) void k_smp_gather(SampleArgs a) {
  __shared__ unsigned int h[256];
  __shared__ int sh_bin;
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int V = a.V;
  const int k = min(a.top_k, V);
  h[tid] = a.hist[(size_t)b * 256 + tid];
  __syncthreads();
  if (tid == 0) {
    int cum = 0, bin = 0;
    for (; bin < 256; ++bin) {
      cum += (int)h[bin];
      if (cum >= k) break;
    }
    sh_bin = bin;  // 256: fewer than k values within 2^24 of the largest (k_sample selects)
  }
  __syncthreads();
  const int b1 = sh_bin;
  if (b1 >= 256) return;
  const float* zr = a.z + (size_t)b * V;
  const uint32_t maxk = a.rowmax[b];
  unsigned long long* cg = a.cand + (size_t)b * SMP_CAND;
  const int v_end = min(V, (int)(blockIdx.x + 1) * SMP_CHUNK);
  for (int v0 = blockIdx.x * SMP_CHUNK; v0 < v_end; v0 += 4 * 256) {
    float zz[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 256 + tid;
      zz[u] = zr[v < v_end ? v : 0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * 256 + tid;
      const uint32_t kk = fkey(zz[u]);
      const uint32_t d = maxk - kk;
      const bool in = v < v_end && d < (1u << 24) && (int)(d >> 16) <= b1;
      const unsigned long long mask = __ballot(in);
      if (mask) {
        const int leader = __ffsll((long long)mask) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(a.ncand + b, __popcll(mask));
        base = __shfl(base, leader, 64);
        const int at = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (in && at < SMP_CAND)
          cg[at] = ((unsigned long long)kk << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)v);
      }
    }
  }
}

// ---- one work-group per row: the top k, min-p, top-p, the draw ---------------------------
__global__ __launch_bounds__(SMP_T) void k_sample(SampleArgs a) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long cand[SMP_CAND];
  __shared__ float cum_s[SMP_T];
  __shared__ float wsum[SMP_T / 64];
  __shared__ int sh_bin, sh_want, sh_n, sh_total;
  __shared__ float sh_u;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int sl = a.row_slot ? a.row_slot[b] : b;
  const int V = a.V;
  float* zr = a.z + (size_t)b * V;
  const int k = min(a.top_k, V);
  if (tid == 0) {
    const unsigned long long w0 = philox_word0((unsigned long long)a.draws[sl], a.seeds[b]);
    sh_u = (float)(unsigned int)(w0 >> 40) * 0x1.0p-24f;
  }
  if (tid < 256) hist[tid] = a.hist[(size_t)b * 256 + tid];
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int i = 0; i < 256; ++i) t += (int)hist[i];
    sh_total = t;
    sh_n = a.ncand[b];
  }
  __syncthreads();
  const uint32_t maxk = a.rowmax[b];
  const bool fast = sh_total >= k && sh_n <= SMP_CAND;
  int nc;
  if (fast) {
    nc = sh_n;
    const unsigned long long* cg = a.cand + (size_t)b * SMP_CAND;
    for (int i = tid; i < nc; i += SMP_T) cand[i] = cg[i];
  } else {
    // exact radix select over the whole scratch row on the distance d = maxk - key of the
    // k-th largest: bins of d >> s over d < 256 << s (s widened until k values fall
    // inside), then 8 bits a pass
    __syncthreads();
    if (tid == 0) sh_n = 0;
    auto count_pass = [&](int shift, uint32_t match_shift, uint32_t match) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int v0 = 0; v0 < V; v0 += SMP_U * SMP_T) {
        float zz[SMP_U];
#pragma unroll
        for (int u = 0; u < SMP_U; ++u) {
          const int v = v0 + u * SMP_T + tid;
          zz[u] = zr[v < V ? v : 0];
        }
#pragma unroll
        for (int u = 0; u < SMP_U; ++u) {
          const int v = v0 + u * SMP_T + tid;
          const uint32_t d = maxk - fkey(zz[u]);
          const bool in = match_shift >= 32 ? (d >> shift) < 256u : (d >> match_shift) == match;
          if (v < V && in) atomicAdd(&hist[(d >> shift) & 0xFFu], 1u);
        }
      }
      __syncthreads();
    };
    auto pick_bin = [&](int want_in) {
      if (tid == 0) {
        int cum = 0, bin = 0;
        for (; bin < 255; ++bin) {
          if (cum + (int)hist[bin] >= want_in) break;
          cum += (int)hist[bin];
        }
        sh_bin = bin;
        sh_want = want_in - cum;
      }
      __syncthreads();
    };
    int s = 16;
    for (;;) {
      count_pass(s, 32u, 0u);
      if (tid == 0) {
        int t = 0;
        for (int i = 0; i < 256; ++i) t += (int)hist[i];
        sh_total = t;
      }
      __syncthreads();
      if (sh_total >= k || s >= 24) break;  // at s = 24 every element is counted
      s += 8;
      __syncthreads();
    }
    pick_bin(k);
    uint32_t dsel = (uint32_t)sh_bin << s;
    int want = sh_want;
    __syncthreads();
    for (int shift = s - 8; shift >= 0; shift -= 8) {
      count_pass(shift, (uint32_t)(shift + 8), dsel >> (shift + 8));
      pick_bin(want);
      dsel |= (uint32_t)sh_bin << shift;
      want = sh_want;
      __syncthreads();
    }
    const uint32_t prefix = maxk - dsel;  // key of the k-th largest value
    // candidates: every key >= the k-th key (ties included), as (key, ~id) for the sort
    for (int v0 = 0; v0 < V; v0 += SMP_U * SMP_T) {
      float zz[SMP_U];
#pragma unroll
      for (int u = 0; u < SMP_U; ++u) {
        const int v = v0 + u * SMP_T + tid;
        zz[u] = zr[v < V ? v : 0];
      }
#pragma unroll
      for (int u = 0; u < SMP_U; ++u) {
        const int v = v0 + u * SMP_T + tid;
        const uint32_t kk = fkey(zz[u]);
        if (v < V && kk >= prefix) {
          const int at = atomicAdd(&sh_n, 1);
          if (at < SMP_CAND) cand[at] = ((unsigned long long)kk << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)v);
        }
      }
    }
    __syncthreads();
    nc = min(sh_n, SMP_CAND);
  }
  __syncthreads();
  // the per-row state is read; clear it for the next call
  if (tid < 256) a.hist[(size_t)b * 256 + tid] = 0u;
  if (tid == 0) {
    a.ncand[b] = 0;
    a.rowmax[b] = 0u;
  }
  int P = 2;
  while (P < nc) P <<= 1;
  for (int i = nc + tid; i < P; i += SMP_T) cand[i] = 0ull;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P / 2; i += SMP_T) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const unsigned long long x = cand[lo], y = cand[hi];
        const bool desc = (lo & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          cand[lo] = y;
          cand[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  // weights relative to the largest, min-p, top-p and the draw over the first n
  const int n = min(k, nc);
  const float z0 = key_value((uint32_t)(cand[0] >> 32));
  float w = 0.0f;
  if (tid < n) w = expf(key_value((uint32_t)(cand[tid] >> 32)) - z0);
  const int n_minp = __syncthreads_count(tid < n && w >= a.min_p);  // a prefix: w is non-increasing
  const float c = block_scan(tid < n_minp ? w : 0.0f, wsum);
  cum_s[tid] = c;
  __syncthreads();
  const float kept = cum_s[n_minp - 1];
  const int below = __syncthreads_count(tid < n_minp && c < a.top_p * kept);
  const int n_topp = min(below + 1, n_minp);
  const float t = sh_u * cum_s[n_topp - 1];
  const int pick = min(__syncthreads_count(tid < n_topp && c <= t), n_topp - 1);
  if (tid == 0) {
    a.next_ids[b] = (int)(0xFFFFFFFFu - (uint32_t)(cand[pick] & 0xFFFFFFFFull));
    a.draws[sl] += 1;
  }
}

// clears the token counts and draw numbers of the slots a prefill is about to fill
__global__ __launch_bounds__(256) void k_reset_seq(int* counts, int* draws, const int* slots, int V) {
  const int sl = slots ? slots[blockIdx.y] : blockIdx.y;
  int* cr = counts + (size_t)sl * V;
  for (int v = blockIdx.x * 1024 + threadIdx.x; v < min(V, (blockIdx.x + 1) * 1024); v += 256) cr[v] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) draws[sl] = 0;
}

hipError_t launch_reset_seq(int* counts, int* draws, const int* slots, int n, int V, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_reset_seq, dim3((V + 1023) / 1024, n), dim3(256), 0, st, counts, draws, slots, V);
  return hipGetLastError();
}

// Per-call scratch of qd_sample_noalloc, for callers that cannot allocate (code under HIP
// graph capture, serving loops that forbid hipMalloc): a fixed array that each device holds
// until the process ends.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol): its device address comes from hipGetSymbolAddress,
// once per device, and the kernels receive that address.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t sample_scratch_address(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

hipError_t launch_sample(const SampleArgs& a, int B, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (a.top_k < 1 || a.top_k > SMP_MAXK) return hipErrorInvalidValue;
  const dim3 g((a.V + SMP_CHUNK - 1) / SMP_CHUNK, B);
  hipLaunchKernelGGL(k_smp_prep, g, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_smp_hist, g, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_smp_gather, g, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_sample, dim3(B), dim3(SMP_T), 0, st, a);
  return hipGetLastError();
}

}  // namespace qd
