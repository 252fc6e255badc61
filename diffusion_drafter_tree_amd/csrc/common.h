// Device helpers shared by the gfx950 kernels of the draft-tree round.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dartree {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Order-preserving map of an fp32 value to an unsigned key: a > b as numbers
// iff key(a) > key(b). -0 is folded onto +0 so that equal numbers tie.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// The same map for bf16 bit patterns (16-bit keys).
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  b &= 0xFFFFu;
  if (b == 0x8000u) b = 0u;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
__device__ __forceinline__ float bf16_key_to_f32(uint32_t k) {
  uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return bf16_to_f32(b);
}

// Split an fp32 value into three bf16 parts by truncation: x == hi + mid + lo
// exactly for normal x (each part keeps the next 8 significant bits).
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  uint32_t u = __float_as_uint(x);
  float fh = __uint_as_float(u & 0xFFFF0000u);
  float r1 = x - fh;
  uint32_t u1 = __float_as_uint(r1);
  float fm = __uint_as_float(u1 & 0xFFFF0000u);
  float r2 = r1 - fm;
  hi = u >> 16;
  mid = u1 >> 16;
  lo = __float_as_uint(r2) >> 16;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, kWave);
    v = v > w ? v : w;
  }
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Exclusive prefix sum across the wave.
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  int lane = lane_id();
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  total = __shfl(x, kWave - 1, kWave);
  return x - v;
}

__device__ __forceinline__ f32x4_t mfma_bf16(const u16x8_t& a, const u16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Block-wide exact top-K of unique 64-bit keys.
//
// Every thread of the block holds EPT keys in registers; 0 marks an empty
// slot (real keys are never 0). On return, out[0..n) holds the n = min(K,
// #keys) largest keys in descending order and out[n..K) is 0. Returns n.
//
// Method: (1) a lower bound tau on the high 32 bits of the K-th largest key:
// each wave whose 64 lanes all hold keys takes the m-th largest of its lane
// maxima, m = ceil(K / number of such waves); the minimum over those waves is
// exceeded by at least K keys. (2) Keys at or above the bound are compacted
// into LDS. (3) Survivors are ranked by counting (small sets) or bitonic
// sorted (larger sets). (4) If more survive than LDS holds, the K-th largest
// key is found exactly by a bitwise search over all 64 bits.
//
// Shared memory: buf[cap] u64, out[K] u64, rank[min(cap, kRankMax)] int,
// misc[8] int. All threads of the block must call it (it synchronises).
// ---------------------------------------------------------------------------
constexpr int kRankMax = 256;

struct TopkSmem {
  uint64_t* buf;
  uint64_t* out;
  int* rank;
  int* misc;
  int cap;
};

template <int EPT>
__device__ int block_topk(const uint64_t (&sk)[EPT], int K, const TopkSmem& sm) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = lane_id();
  const int nwave = nthr / kWave;
  int* misc = sm.misc;
  // misc: 0 full waves, 1 total keys, 2 tau (min), 3 survivors, 4 tau set flag
  if (tid == 0) {
    misc[0] = 0; misc[1] = 0; misc[2] = -1; misc[3] = 0; misc[4] = 0; misc[5] = 0;
  }
  __syncthreads();
  uint32_t lmax = 0;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    uint32_t hi = (uint32_t)(sk[e] >> 32);
    lmax = hi > lmax ? hi : lmax;
    cnt += sk[e] != 0ull;
  }
  uint64_t valid = __ballot(lmax != 0u);
  bool full = valid == ~0ull;
  int wcnt = wave_sum_i32(cnt);
  if (lane == 0) {
    if (full) atomicAdd(&misc[0], 1);
    atomicAdd(&misc[1], wcnt);
  }
  __syncthreads();
  const int nwf = misc[0];
  const int ntot = misc[1];
  (void)nwave;
  if (nwf > 0) {
    int m = (K + nwf - 1) / nwf;
    if (m <= kWave && full) {
      // m-th largest lane maximum of this wave, bit by bit from the top
      uint32_t t = 0;
      for (int b = 31; b >= 0; --b) {
        uint32_t c = t | (1u << b);
        int n = __popcll(__ballot(lmax >= c));
        if (n >= m) t = c;
      }
      if (lane == 0) {
        atomicMin(reinterpret_cast<unsigned int*>(&misc[2]), t);
        atomicOr(&misc[4], 1);
      }
    }
  }
  __syncthreads();
  const uint64_t thr = misc[4] ? ((uint64_t)(uint32_t)misc[2] << 32) : 1ull;
  // compaction of survivors
  int c2 = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) c2 += (sk[e] != 0ull && sk[e] >= thr);
  int wtot;
  int pre = wave_excl_scan(c2, wtot);
  int base = 0;
  if (lane == 0 && wtot) base = atomicAdd(&misc[3], wtot);
  base = __shfl(base, 0, kWave);
  int pos = base + pre;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (sk[e] != 0ull && sk[e] >= thr) {
      if (pos < sm.cap) sm.buf[pos] = sk[e];
      ++pos;
    }
  }
  __syncthreads();
  int ns = misc[3];
  if (ns > sm.cap) {
    // Exact K-th largest key by a bitwise search (rare: massive ties).
    uint64_t T = 0;
    int need = K < ntot ? K : ntot;
    for (int b = 63; b >= 0; --b) {
      uint64_t c = T | (1ull << b);
      int n = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) n += (sk[e] != 0ull && sk[e] >= c);
      n = wave_sum_i32(n);
      if (tid == 0) misc[5] = 0;
      __syncthreads();
      if (lane == 0 && n) atomicAdd(&misc[5], n);
      __syncthreads();
      if (misc[5] >= need) T = c;
      __syncthreads();
    }
    if (tid == 0) misc[3] = 0;
    __syncthreads();
    c2 = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) c2 += (sk[e] != 0ull && sk[e] >= T);
    pre = wave_excl_scan(c2, wtot);
    base = 0;
    if (lane == 0 && wtot) base = atomicAdd(&misc[3], wtot);
    base = __shfl(base, 0, kWave);
    pos = base + pre;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (sk[e] != 0ull && sk[e] >= T) {
        if (pos < sm.cap) sm.buf[pos] = sk[e];
        ++pos;
      }
    }
    __syncthreads();
    ns = misc[3];
  }
  const int n_out = ns < K ? ns : K;
  if (ns <= kRankMax) {
    // rank by counting: rank(i) = #{j : buf[j] > buf[i]}
    for (int i = tid; i < ns; i += nthr) sm.rank[i] = 0;
    __syncthreads();
    if (ns > 0) {
      int nseg = nthr / ns;
      if (nseg < 1) nseg = 1;
      int seg = (ns + nseg - 1) / nseg;
      for (int t = tid; t < ns * nseg; t += nthr) {
        int i = t % ns, s = t / ns;
        uint64_t x = sm.buf[i];
        int j0 = s * seg, j1 = min(ns, j0 + seg);
        int r = 0;
        for (int j = j0; j < j1; ++j) r += sm.buf[j] > x;
        if (r) atomicAdd(&sm.rank[i], r);
      }
    }
    __syncthreads();
    for (int i = tid; i < ns; i += nthr) {
      int r = sm.rank[i];
      if (r < K) sm.out[r] = sm.buf[i];
    }
    for (int i = n_out + tid; i < K; i += nthr) sm.out[i] = 0ull;
    __syncthreads();
  } else {
    int P = 1;
    while (P < ns) P <<= 1;
    for (int i = ns + tid; i < P; i += nthr) sm.buf[i] = 0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < (P >> 1); i += nthr) {
          int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
          int hi = lo + j;
          bool desc = (lo & k) == 0;
          uint64_t x = sm.buf[lo], y = sm.buf[hi];
          if ((x < y) == desc) { sm.buf[lo] = y; sm.buf[hi] = x; }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < K; i += nthr) sm.out[i] = i < n_out ? sm.buf[i] : 0ull;
    __syncthreads();
  }
  return n_out;
}

}  // namespace dartree
