// Step a1 (per-position top-K candidates) and step a0 (head inputs) in one
// launch.
//
// DARTree (marsggbo blog, section 3.1): every block position keeps its K best
// tokens of the drafter's base logits (value descending, token id ascending);
// a block-parallel drafter forward provides H_d, here projected to h_d.
//
// Scan workgroups (1024 threads): one per (row, slice) of logits[rows][V]. A
// slice is held in registers (up to NV 16-byte vectors per thread). The
// values are scanned as signed 16-bit (bf16) or 32-bit (fp32) integers: for
// positive numbers that order equals the numeric order and negative numbers
// sort below every positive one, so packed integer max and compare work on
// the raw bits. Each wave takes the m-th largest positive lane maximum, m =
// ceil(K / 16), and the smallest of those is a lower bound exceeded by at
// least K elements; only elements at or above it become 64-bit sort keys and
// go through the exact selection. Rows where the bound does not hold
// (fewer than m positive lanes in a wave, or more survivors than fit) take an
// exact path: a bitwise search for the K-th largest value and an id-ordered
// choice among values equal to it.
//
// Head workgroups: one per 16x16 tile of h[M][r] = H[M][D] * P[D][r] (Pt
// stored [r][D]); the 16 waves split D, each issuing all its loads before its
// v_mfma_f32_16x16x32_bf16 instructions, and the partial tiles are added in a
// fixed order.
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / kWave;
constexpr int kScanCap = 1024;

struct ScanSmem {
  uint64_t key[kScanCap];
  int pay[kScanCap];
  int rank[kScanCap];
  uint64_t out_key[1024];
  int out_pay[1024];
  int misc[8];
  int wsum[kWaves];
};
struct HeadSmem {
  float part[kWaves][16][17];
};
union KernelSmem {
  ScanSmem scan;
  HeadSmem head;
};

template <bool BF16>
struct Traits;
template <>
struct Traits<true> {
  static constexpr int EPV = 8;   // elements per 16-byte vector
  static constexpr int KBITS = 16;
  __device__ static uint32_t raw(const u32x4_t& q, int e) { return (q[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu; }
  __device__ static int sval(uint32_t raw) { return (int)(int16_t)(uint16_t)raw; }   // signed view
  __device__ static uint32_t key(uint32_t raw) { return bf16_key(raw); }
  __device__ static float value(uint32_t key) { return bf16_key_to_f32(key); }
  // signed max of the 8 lanes of a vector (packed 16-bit max). The words are
  // taken from a local copy by name: bit-casting subscripted elements of a
  // vector reference was seen to drop all but the first word.
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  __device__ static s16x2_t as_s16x2(unsigned int x) { return __builtin_bit_cast(s16x2_t, x); }
  __device__ static int vmax(u32x4_t q) {
    const s16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(as_s16x2(q.x), as_s16x2(q.y)),
                                                 __builtin_elementwise_max(as_s16x2(q.z), as_s16x2(q.w)));
    return max((int)m2.x, (int)m2.y);
  }
  __device__ static u32x4_t neg_fill() { return u32x4_t{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}; }
};
template <>
struct Traits<false> {
  static constexpr int EPV = 4;
  static constexpr int KBITS = 32;
  __device__ static uint32_t raw(const u32x4_t& q, int e) { return q[e]; }
  __device__ static int sval(uint32_t raw) { return (int)raw; }
  __device__ static uint32_t key(uint32_t raw) { return f32_key(__uint_as_float(raw)); }
  __device__ static float value(uint32_t key) { return key_to_f32(key); }
  __device__ static int vmax(u32x4_t q) { return max(max((int)q.x, (int)q.y), max((int)q.z, (int)q.w)); }
  __device__ static u32x4_t neg_fill() { return u32x4_t{0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u}; }
};

// rank-count selection over ns keys already in sm.key/sm.pay (ns <= cap)
__device__ int lds_rank_select(ScanSmem& sm, int ns, int K) {
  const int tid = threadIdx.x;
  if (ns > 0) {
    int nseg = kT / ns;
    if (nseg < 1) nseg = 1;
    const int seg = (ns + nseg - 1) / nseg;
    for (int t = tid; t < ns * nseg; t += kT) {
      const int i = t % ns, s = t / ns;
      const uint64_t x = sm.key[i];
      const int j0 = s * seg, j1 = min(ns, j0 + seg);
      int r = 0;
      for (int j = j0; j < j1; ++j) r += sm.key[j] > x;
      if (r) atomicAdd(&sm.rank[i], r);
    }
  }
  __syncthreads();
  const int n_out = min(ns, K);
  for (int i = tid; i < ns; i += kT) {
    const int r = sm.rank[i];
    if (r < K) sm.out_key[r] = sm.key[i];
  }
  for (int i = n_out + tid; i < K; i += kT) sm.out_key[i] = 0ull;
  __syncthreads();
  return n_out;
}

// Block-wide sum of an int (every thread gets the total). Two barriers.
__device__ int block_sum(ScanSmem& sm, int v) {
  const int w = threadIdx.x / kWave;
  const int s = wave_sum_i32(v);
  if (lane_id() == 0) sm.wsum[w] = s;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += sm.wsum[i];
  __syncthreads();
  return t;
}

template <bool BF16, int NV>
__device__ void scan_block(const ScanArgs& a, ScanSmem& sm, int blk) {
  using Tr = Traits<BF16>;
  constexpr int EPV = Tr::EPV;
  constexpr int ESZ = 16 / EPV;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int row = blk / a.S, sl = blk - row * a.S;
  const int s0 = sl * a.slice;
  const int s1 = min(a.V, s0 + a.slice);
  const char* rowp = static_cast<const char*>(a.logits) + (size_t)row * (size_t)a.V * ESZ;
  const bool vec_ok = (((uintptr_t)rowp) & 15u) == 0;
  const int K = a.K;

  // -- load the slice: vector it of thread t covers elements s0 + (it*kT + t)*EPV ..
  u32x4_t q[NV];
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    const int e0 = s0 + (it * kT + tid) * EPV;
    if (vec_ok && e0 + EPV <= s1) {
      q[it] = *reinterpret_cast<const u32x4_t*>(rowp + (size_t)e0 * ESZ);
    } else {
      uint32_t wv[4];
      const u32x4_t nf = Tr::neg_fill();
      wv[0] = nf.x; wv[1] = nf.y; wv[2] = nf.z; wv[3] = nf.w;
      if (e0 < s1) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          if (e0 + e < s1) {
            const uint32_t r = BF16 ? (uint32_t)(reinterpret_cast<const uint16_t*>(rowp)[e0 + e])
                                    : reinterpret_cast<const uint32_t*>(rowp)[e0 + e];
            if (BF16)
              wv[e >> 1] = (wv[e >> 1] & ~(0xFFFFu << ((e & 1) * 16))) | (r << ((e & 1) * 16));
            else
              wv[e] = r;
          }
        }
      }
      q[it] = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
    }
  }
  // -- lane maxima on the signed view (positive values order correctly)
  int vm[NV];
  int lmax = -0x7FFFFFFF;
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    vm[it] = Tr::vmax(q[it]);
    lmax = max(lmax, vm[it]);
  }
  // -- bound: each active wave's m-th largest positive lane maximum. A wave
  //    is active when its first lane holds an element of the slice.
  const int nthr_valid = min(kT, (s1 - s0 + EPV - 1) / EPV);
  const int nact = (nthr_valid + kWave - 1) / kWave;
  const int m = (K + nact - 1) / nact;
  if (w < nact) {
    const bool pos = lmax > 0;
    const int npos = __popcll(__ballot(pos));
    if (npos >= m && m <= kWave) {
      const uint32_t t = wave_mth_largest((uint32_t)lmax, pos, m, Tr::KBITS == 16 ? 15 : 31);
      if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(&sm.misc[2]), ~t);
    } else if (lane == 0) {
      atomicOr(&sm.misc[4], 1);   // this wave cannot vouch for m elements
    }
  }
  for (int i = tid; i < kScanCap; i += kT) sm.rank[i] = 0;
  __syncthreads();
  const bool bound_ok = sm.misc[4] == 0;
  const int tau = (int)(~(uint32_t)sm.misc[2]);
  int ns = kScanCap + 1;
  if (bound_ok) {
    // -- survivors: elements with signed value >= tau (tau > 0)
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const uint64_t hit = __ballot(vm[it] >= tau);
      if (hit) {
        const int e0 = s0 + (it * kT + tid) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const uint32_t r = Tr::raw(q[it], e);
          const bool sv = ((hit >> lane) & 1ull) && Tr::sval(r) >= tau && e0 + e < s1;
          const uint64_t b = __ballot(sv);
          if (b) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&sm.misc[3], __popcll(b));
            base = __builtin_amdgcn_readfirstlane(base);
            if (sv) {
              const int p = base + (int)mbcnt64(b);
              if (p < kScanCap) sm.key[p] = ((uint64_t)Tr::key(r) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(e0 + e));
            }
          }
        }
      }
    }
    __syncthreads();
    ns = sm.misc[3];
  }
  if (!bound_ok || ns > kScanCap) {
    // -- exact path: K-th largest value key by a bitwise search, then the
    //    keys above it and the lowest ids among the keys equal to it
    int nvalid = 0;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e0 = s0 + (it * kT + tid) * EPV;
      nvalid += max(0, min(EPV, s1 - e0));
    }
    const int need = min(K, block_sum(sm, nvalid));
    uint32_t T = 0;
    for (int b = Tr::KBITS - 1; b >= 0; --b) {
      const uint32_t c = T | (1u << b);
      int n = 0;
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e0 = s0 + (it * kT + tid) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) n += (e0 + e < s1 && Tr::key(Tr::raw(q[it], e)) >= c);
      }
      if (block_sum(sm, n) >= need) T = c;
    }
    // keys strictly above T (fewer than need), in any order
    if (tid == 0) sm.misc[3] = 0;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e0 = s0 + (it * kT + tid) * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const uint32_t kk = Tr::key(Tr::raw(q[it], e));
        if (e0 + e < s1 && kk > T) {
          const int p = atomicAdd(&sm.misc[3], 1);
          sm.key[p] = ((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(e0 + e));
        }
      }
    }
    __syncthreads();
    const int ngt = sm.misc[3];
    int take = need - ngt;   // keys equal to T, lowest ids first
    // ids grow with (it, thread, e): walk the vector rounds in order
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e0 = s0 + (it * kT + tid) * EPV;
      int c = 0;
#pragma unroll
      for (int e = 0; e < EPV; ++e) c += (e0 + e < s1 && Tr::key(Tr::raw(q[it], e)) == T);
      // exclusive prefix of c over threads in tid order
      const int wtot = wave_sum_i32(c);
      uint32_t x = (uint32_t)c;   // inclusive scan within the wave by shifts
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, o, kWave);
        if (lane >= o) x += y;
      }
      if (lane == 0) sm.wsum[w] = wtot;
      __syncthreads();
      int before = 0, all = 0;
      for (int i = 0; i < kWaves; ++i) {
        before += i < w ? sm.wsum[i] : 0;
        all += sm.wsum[i];
      }
      int r = before + (int)x - c;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const uint32_t kk = Tr::key(Tr::raw(q[it], e));
        if (e0 + e < s1 && kk == T) {
          if (r < take) sm.key[ngt + (need - ngt - take) + r] =
              ((uint64_t)kk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(e0 + e));
          ++r;
        }
      }
      __syncthreads();
      take -= min(all, take);   // 0 once every needed key is taken; later rounds write nothing
    }
    ns = need;
    __syncthreads();
  }
  const int n = lds_rank_select(sm, ns, K);
  (void)n;
  if (a.S == 1) {
    int32_t* ids = a.cand_ids + (size_t)row * K;
    float* vals = a.cand_logit + (size_t)row * K;
    for (int i = tid; i < K; i += kT) {
      const uint64_t x = sm.out_key[i];
      ids[i] = x ? (int32_t)(0xFFFFFFFFu - (uint32_t)x) : -1;
      vals[i] = x ? Tr::value((uint32_t)(x >> 32)) : -__builtin_huge_valf();
    }
  } else {
    uint64_t* lst = a.lists + ((size_t)row * a.S + sl) * K;
    for (int i = tid; i < K; i += kT) lst[i] = sm.out_key[i];
  }
}

__device__ void head_block(const ScanArgs& a, HeadSmem& sm, int tile) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int ntn = a.r / 16;
  const int nt = tile % ntn, mt = tile / ntn;
  const int KS = a.D / 32;
  const int k0 = (KS * w) / kWaves, k1 = (KS * (w + 1)) / kWaves;
  const int m = mt * 16 + (lane & 15);
  const int n = nt * 16 + (lane & 15);
  const int sub = (lane >> 4) * 8;
  const uint16_t* hrow = a.H + (size_t)(m < a.M ? m : 0) * a.D + sub;
  const uint16_t* prow = a.Pt + (size_t)n * a.D + sub;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int G = 8;
  for (int kb = k0; kb < k1; kb += G) {
    u16x8_t av[G], bv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (kb + g < k1) {
        av[g] = *reinterpret_cast<const u16x8_t*>(hrow + (kb + g) * 32);
        bv[g] = *reinterpret_cast<const u16x8_t*>(prow + (kb + g) * 32);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (kb + g < k1) {
        if (m >= a.M) av[g] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        acc = mfma_bf16(av[g], bv[g], acc);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.part[w][(lane >> 4) * 4 + i][lane & 15] = acc[i];
  __syncthreads();
  if (w < 4) {
    const int rr = w * 4 + (lane >> 4), cc = lane & 15;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) v += sm.part[i][rr][cc];
    const int mm = mt * 16 + rr;
    if (mm < a.M) a.h[(size_t)mm * a.r + nt * 16 + cc] = v;
  }
}

template <bool BF16, int NV>
__global__ __launch_bounds__(kT) void scan_kernel(ScanArgs a) {
  __shared__ KernelSmem smem;
  const int b = blockIdx.x;
  if (b < a.n_scan) {
    if (threadIdx.x < 8) smem.scan.misc[threadIdx.x] = 0;
    __syncthreads();
    scan_block<BF16, NV>(a, smem.scan, b);
  } else {
    head_block(a, smem.head, b - a.n_scan);
  }
}

// Per-row merge of S sorted slice lists (used when a row spans several slices).
template <int EPT>
__global__ __launch_bounds__(kT) void merge_kernel(const uint64_t* __restrict__ lists, int S, int K, bool bf16,
                                                   int32_t* __restrict__ cand_ids, float* __restrict__ cand_logit) {
  __shared__ uint64_t s_key[kScanCap];
  __shared__ int s_pay[kScanCap];
  __shared__ int s_rank[kScanCap];
  __shared__ uint64_t s_out[1024];
  __shared__ int s_outp[1024];
  __shared__ int s_misc[8];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (tid < 8) s_misc[tid] = 0;
  for (int i = tid; i < kScanCap; i += kT) s_rank[i] = 0;
  __syncthreads();
  const uint64_t* L = lists + (size_t)row * S * K;
  uint64_t k[EPT];
  int p[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid + e * kT;
    k[e] = i < S * K ? L[i] : 0ull;
    p[e] = 0;
  }
  SelSmem sm{(LDS uint64_t*)s_key, (LDS int*)s_pay, (LDS int*)s_rank, (LDS uint64_t*)s_out, (LDS int*)s_outp,
             (LDS int*)s_misc, kScanCap};
  block_select<EPT>(k, p, K, bf16 ? 16 : 32, sm);
  for (int i = tid; i < K; i += kT) {
    const uint64_t x = s_out[i];
    cand_ids[(size_t)row * K + i] = x ? (int32_t)(0xFFFFFFFFu - (uint32_t)x) : -1;
    cand_logit[(size_t)row * K + i] =
        x ? (bf16 ? bf16_key_to_f32((uint32_t)(x >> 32)) : key_to_f32((uint32_t)(x >> 32))) : -__builtin_huge_valf();
  }
}

__global__ __launch_bounds__(256) void head_valu_f32(const float* __restrict__ H, const float* __restrict__ Pt,
                                                     float* __restrict__ h, int M, int D, int r) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * r) return;
  const int m = (int)(idx / r), j = (int)(idx % r);
  float acc = 0.f;
  for (int i = 0; i < D; ++i) acc = fmaf(H[(size_t)m * D + i], Pt[(size_t)j * D + i], acc);
  h[idx] = acc;
}
__global__ __launch_bounds__(256) void head_valu_bf16(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Pt,
                                                      float* __restrict__ h, int M, int D, int r) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * r) return;
  const int m = (int)(idx / r), j = (int)(idx % r);
  float acc = 0.f;
  for (int i = 0; i < D; ++i) acc = fmaf(bf16_to_f32(H[(size_t)m * D + i]), bf16_to_f32(Pt[(size_t)j * D + i]), acc);
  h[idx] = acc;
}

constexpr int kNvOptions[] = {2, 4, 8, 12, 16, 20};

}  // namespace

ScanPlan scan_plan(int rows, int V, int K, bool bf16) {
  ScanPlan p{};
  const int epv = bf16 ? 8 : 4;
  const int max_nv = 20;
  // slices per row: as few as fit in registers (max_nv vectors per thread)
  const long long per_wg = (long long)kT * epv * max_nv;
  p.S = (int)((V + per_wg - 1) / per_wg);
  // slice length: multiple of the vector width
  long long sl = ((long long)V + p.S - 1) / p.S;
  sl = (sl + epv - 1) / epv * epv;
  p.slice = (int)sl;
  const int nvec = (int)((sl + epv - 1) / epv);
  const int need_nv = (nvec + kT - 1) / kT;
  p.nv = 0;
  for (int o : kNvOptions)
    if (o >= need_nv) { p.nv = o; break; }
  p.n_scan = rows * p.S;
  p.merge_ept = (p.S * K + kT - 1) / kT <= 8 ? 8 : 16;
  p.list_bytes = p.S > 1 ? (size_t)rows * p.S * K * sizeof(uint64_t) : 0;
  p.ok = p.nv > 0 && (long long)p.S * K <= 16LL * kT;
  return p;
}

bool head_mfma_ok(bool bf16, const void* H, const void* Pt, int D, int r) {
  return bf16 && D % 32 == 0 && r % 16 == 0 && ((((uintptr_t)H) | ((uintptr_t)Pt)) & 15u) == 0;
}

hipError_t launch_scan(const ScanPlan& p, bool bf16, const ScanArgs& args_in, hipStream_t s) {
  ScanArgs a = args_in;
  a.S = p.S;
  a.slice = p.slice;
  a.n_scan = p.n_scan;
  const int grid = a.n_scan + a.n_head;
  if (grid == 0) return hipSuccess;
#define DT_SCAN(B, NVV) hipLaunchKernelGGL((scan_kernel<B, NVV>), dim3(grid), dim3(kT), 0, s, a)
  switch (p.nv) {
    case 2: if (bf16) DT_SCAN(true, 2); else DT_SCAN(false, 2); break;
    case 4: if (bf16) DT_SCAN(true, 4); else DT_SCAN(false, 4); break;
    case 8: if (bf16) DT_SCAN(true, 8); else DT_SCAN(false, 8); break;
    case 12: if (bf16) DT_SCAN(true, 12); else DT_SCAN(false, 12); break;
    case 16: if (bf16) DT_SCAN(true, 16); else DT_SCAN(false, 16); break;
    default: if (bf16) DT_SCAN(true, 20); else DT_SCAN(false, 20); break;
  }
#undef DT_SCAN
  return hipGetLastError();
}

hipError_t launch_merge(const ScanPlan& p, int rows, int K, bool bf16, const uint64_t* lists, int32_t* cand_ids,
                        float* cand_logit, hipStream_t s) {
  if (p.S <= 1) return hipSuccess;
  if (p.merge_ept == 8)
    hipLaunchKernelGGL((merge_kernel<8>), dim3(rows), dim3(kT), 0, s, lists, p.S, K, bf16, cand_ids, cand_logit);
  else
    hipLaunchKernelGGL((merge_kernel<16>), dim3(rows), dim3(kT), 0, s, lists, p.S, K, bf16, cand_ids, cand_logit);
  return hipGetLastError();
}

hipError_t launch_head(bool bf16, const void* H, const void* Pt, float* h, int M, int D, int r, hipStream_t s) {
  if (!head_mfma_ok(bf16, H, Pt, D, r)) return launch_head_valu(bf16, H, Pt, h, M, D, r, s);
  ScanArgs a{};
  a.H = static_cast<const uint16_t*>(H);
  a.Pt = static_cast<const uint16_t*>(Pt);
  a.h = h;
  a.M = M;
  a.D = D;
  a.r = r;
  a.n_head = (r / 16) * ((M + 15) / 16);
  a.n_scan = 0;
  hipLaunchKernelGGL((scan_kernel<true, 2>), dim3(a.n_head), dim3(kT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_head_valu(bool bf16, const void* H, const void* Pt, float* h, int M, int D, int r, hipStream_t s) {
  const size_t total = (size_t)M * r;
  dim3 grid((unsigned)((total + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(head_valu_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(H),
                       static_cast<const uint16_t*>(Pt), h, M, D, r);
  else
    hipLaunchKernelGGL(head_valu_f32, grid, dim3(256), 0, s, static_cast<const float*>(H),
                       static_cast<const float*>(Pt), h, M, D, r);
  return hipGetLastError();
}

}  // namespace dartree
