// Step a1 (per-position top-K candidates) and step a0 (head inputs) in one
// launch.
//
// DARTree (marsggbo blog, section 3.1): every block position keeps its K best
// tokens of the drafter's base logits (value descending, token id ascending);
// a block-parallel drafter forward provides H_d, here projected to h_d.
//
// Scan workgroups (1024 threads): one per (row, slice) of logits[rows][V]; a
// thread holds at most five 16-byte vectors of its slice in registers. Values
// are compared as ordered integer keys (bf16: 16 bits, fp32: 32 bits, -0 and
// +0 equal). A vector's largest key comes from a packed signed max and min of
// its raw bits (the signed view orders non-negative values and reverses
// negative ones). Each wave takes the m-th largest of its lanes' largest keys,
// m = ceil(K / active waves); the smallest of those, T, is reached by at least
// K elements. Vectors holding a key >= T are queued in LDS (one LDS atomic
// per wave), their elements checked one a thread and the survivors compacted
// (one LDS atomic per wave and pass), then ranked by counting, G threads per
// survivor (bf16: on 32-bit keys, two survivors a group). A slice whose bound
// fails (a wave with fewer than m lanes) or whose survivors overflow takes an
// exact path: bitwise searches for the K-th largest key and, among keys equal
// to it, for the largest complemented ids.
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
constexpr int kScanCap = 2048;   // survivors a slice may hold
constexpr int kMaxNV = 5;        // 16-byte vectors per thread

constexpr int kHitCap = 512;     // vectors holding a key >= T
struct ScanSmem {
  uint64_t key[kScanCap + 8];
  uint32_t key32[kScanCap + 32];   // bf16 slices: 32-bit survivor keys, zero-padded
  uint64_t out[1024];
  u32x4_t hitq[kHitCap];
  int hitid[kHitCap];
  int bhist[256];   // lane maxima by distance below the slice's largest key
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

// Wide variant (K > 64), NT threads a workgroup: the hit queue holds 2 NT
// vectors and the survivor list 4 NT 32-bit keys (bf16; half as many 64-bit
// keys for fp32); the hit queue's space is reused for the histogram
// selection's buckets and output once the queued vectors have been checked.
#ifndef DARTREE_WIDE_NT
#define DARTREE_WIDE_NT 1024
#endif
constexpr int kWideT = DARTREE_WIDE_NT;
template <int NT>
struct WideSmem {
  static constexpr int kHit = 2 * NT, kSurv = 4 * NT;
  union {
    struct {
      u32x4_t hitq[kHit];
      int hitid[kHit];
    };
    struct {
      uint64_t bucket[kSurv];
      uint64_t out[1024];
    };
  };
  union {
    uint32_t key32[kSurv + 32];
    uint64_t key[kSurv / 2 + 8];
  };
  int hist[256];
  int cursor[256];
  int base[256];
  int bhist[256];   // lane maxima by distance below the slice's largest key
  int misc[8];
  int wsum[NT / kWave];
};
// Head tiles for many rows: 64 x 64 outputs per workgroup, D staged through
// LDS in double-buffered stages of 128 columns (rows padded by 8 elements).
constexpr int kHB = 64, kHS = 128, kHP = kHS + 8;
struct HeadBigSmem {
  uint16_t a[2][kHB][kHP];
  uint16_t b[2][kHB][kHP];
};
static_assert(sizeof(HeadBigSmem) >= 4 * kHB * (kHB + 1) * sizeof(float), "partial quadrants fit the staging buffers");
template <int NT>
union WideKernelSmem {
  WideSmem<NT> scan;
  HeadSmem head;
  HeadBigSmem headbig;
};

template <bool BF16>
struct Traits;
template <>
struct Traits<true> {
  static constexpr int EPV = 8;   // elements per 16-byte vector
  static constexpr int KBITS = 16;
  __device__ static uint32_t raw(u32x4_t q, int e) {
    const uint32_t w = e < 2 ? q.x : e < 4 ? q.y : e < 6 ? q.z : q.w;
    return (w >> ((e & 1) * 16)) & 0xFFFFu;
  }
  __device__ static uint32_t key(uint32_t raw) { return bf16_key(raw); }
  __device__ static float value(uint32_t key) { return bf16_key_to_f32(key); }
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  __device__ static s16x2_t as_s16x2(unsigned int x) { return __builtin_bit_cast(s16x2_t, x); }
  // largest key of the 8 values (words taken by name from a local copy)
  __device__ static uint32_t vec_key_max(u32x4_t q) {
    const s16x2_t a = as_s16x2(q.x), b = as_s16x2(q.y), c = as_s16x2(q.z), d = as_s16x2(q.w);
    const s16x2_t mx = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    const s16x2_t mn = __builtin_elementwise_min(__builtin_elementwise_min(a, b), __builtin_elementwise_min(c, d));
    const int smax = max((int)mx.x, (int)mx.y), smin = min((int)mn.x, (int)mn.y);
    return smax >= 0 ? 0x8000u + (uint32_t)smax : (uint32_t)(-smin);
  }
  __device__ static uint32_t fill_word() { return 0xFFFFFFFFu; }   // key 1 per element, the lowest
};
template <>
struct Traits<false> {
  static constexpr int EPV = 4;
  static constexpr int KBITS = 32;
  __device__ static uint32_t raw(u32x4_t q, int e) { return e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w; }
  __device__ static uint32_t key(uint32_t raw) { return f32_key(__uint_as_float(raw)); }
  __device__ static float value(uint32_t key) { return key_to_f32(key); }
  __device__ static uint32_t vec_key_max(u32x4_t q) {
    const int smax = max(max((int)q.x, (int)q.y), max((int)q.z, (int)q.w));
    const int smin = min(min((int)q.x, (int)q.y), min((int)q.z, (int)q.w));
    return smax >= 0 ? (0x80000000u | (uint32_t)smax) : (smin == (int)0x80000000 ? 0x80000000u : ~(uint32_t)smin);
  }
  __device__ static uint32_t fill_word() { return 0xFFFFFFFFu; }   // key 0, the lowest
};

// Block-wide sum of an int (every thread gets the total). Two barriers.
template <class Smem>
__device__ int block_sum(Smem& sm, int v) {
  constexpr int kWaves = sizeof(sm.wsum) / sizeof(sm.wsum[0]);
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

// Ranks the ns distinct keys in sm.key by counting, G threads per key, and
// writes the K largest in descending order to sm.out (zero beyond ns).
__device__ void rank_select(ScanSmem& sm, int ns, int K) {
  const int tid = threadIdx.x;
  int G = 16;
  while (G > 1 && ns * G > kT) G >>= 1;
  const int per = (((ns + G - 1) / G) + 7) & ~7;   // multiple of 8: 16-byte aligned segments
  for (int x0 = 0; x0 < ns; x0 += kT / G) {
    const int x = x0 + tid / G, seg = tid % G;
    uint64_t kx = 0ull;
    uint32_t cnt = 0u;
    if (x < ns) {
      kx = sm.key[x];
      const int y1 = min(ns, (seg + 1) * per);
      for (int y = seg * per; y < y1; y += 8) {
        uint64_t k8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) k8[e] = sm.key[y + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) cnt += (y + e < y1 && k8[e] > kx) ? 1u : 0u;
      }
    }
    if (G >= 2) cnt += dpp<kDppXor1>(cnt);
    if (G >= 4) cnt += dpp<kDppXor2>(cnt);
    if (G >= 8) cnt += lane_xor<4>(cnt);
    if (G >= 16) cnt += lane_xor<8>(cnt);
    if (x < ns && seg == 0 && (int)cnt < K) sm.out[cnt] = kx;
  }
  for (int i = ns + tid; i < K; i += kT) sm.out[i] = 0ull;
  __syncthreads();
}

// The same for bf16 slices on 32-bit keys (bf16 key << 16 | 0xFFFF - offset
// in the slice: slices are shorter than 65,536 elements, so the keys are
// distinct and in the same order as the 64-bit ones). A group of G threads
// ranks two survivors (x and x + ceil(ns / 2)) against one segment of the
// keys, read eight at a time (the segments are as short as the group
// allows: every lane of a wave pays for its busiest lane's compares); keys
// past ns are zero, so segments are read in whole steps. The output is the
// 64-bit form.
static_assert(kT * 8 * kMaxNV <= 65536 && kWideT * 8 * kMaxNV <= 65536,
              "a bf16 slice must fit the 16-bit offset of its 32-bit survivor keys");
__device__ void rank_select32(ScanSmem& sm, int ns, int K, int s0) {
  const int tid = threadIdx.x;
  const int ng = (ns + 1) >> 1;
  int G = 16;
  while (G > 1 && ng * G > kT) G >>= 1;
  const int per = (((ns + G - 1) / G) + 7) & ~7;   // multiple of 8
  auto out64 = [&](uint32_t k) {
    const uint32_t idx = (uint32_t)s0 + 0xFFFFu - (k & 0xFFFFu);
    return ((uint64_t)(k >> 16) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
  };
  for (int g0 = 0; g0 < ng; g0 += kT / G) {
    const int g = g0 + tid / G, seg = tid % G;
    const int xb = g + ng;
    uint32_t ka = 0u, kb = 0u, ca = 0u, cb = 0u;
    if (g < ng) {
      ka = sm.key32[g];
      kb = sm.key32[xb];   // xb <= ns: the zero pad when ns is odd (unused)
      const int y1 = min(ns, (seg + 1) * per);
      for (int y = seg * per; y < y1; y += 8) {
        u32x4_t k4[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) k4[e] = *reinterpret_cast<const u32x4_t*>(&sm.key32[y + 4 * e]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          ca += (k4[e].x > ka ? 1u : 0u) + (k4[e].y > ka ? 1u : 0u) + (k4[e].z > ka ? 1u : 0u) + (k4[e].w > ka ? 1u : 0u);
          cb += (k4[e].x > kb ? 1u : 0u) + (k4[e].y > kb ? 1u : 0u) + (k4[e].z > kb ? 1u : 0u) + (k4[e].w > kb ? 1u : 0u);
        }
      }
    }
    if (G >= 2) { ca += dpp<kDppXor1>(ca); cb += dpp<kDppXor1>(cb); }
    if (G >= 4) { ca += dpp<kDppXor2>(ca); cb += dpp<kDppXor2>(cb); }
    if (G >= 8) { ca += lane_xor<4>(ca); cb += lane_xor<4>(cb); }
    if (G >= 16) { ca += lane_xor<8>(ca); cb += lane_xor<8>(cb); }
    if (g < ng && seg == 0) {
      if ((int)ca < K) sm.out[ca] = out64(ka);
      if (xb < ns && (int)cb < K) sm.out[cb] = out64(kb);
    }
  }
  for (int i = ns + tid; i < K; i += kT) sm.out[i] = 0ull;
  __syncthreads();
}

// The slice blk of the logits into q: at most kMaxNV 16-byte vectors per
// thread; absent elements get the lowest key.
template <bool BF16, int NV, int kT>
__device__ __forceinline__ void load_slice(const ScanArgs& a, int blk, u32x4_t (&q)[NV]) {
  using Tr = Traits<BF16>;
  constexpr int EPV = Tr::EPV;
  constexpr int ESZ = 16 / EPV;
  const int tid = threadIdx.x;
  const int row = blk / a.S, sl = blk - row * a.S;
  const int s0 = sl * a.slice;
  const int s1 = min(a.V, s0 + a.slice);
  const char* rowp = static_cast<const char*>(a.logits) + (size_t)row * (size_t)a.V * ESZ;
  const bool vec_ok = (((uintptr_t)rowp) & 15u) == 0;
  auto id0 = [&](int it) { return s0 + (it * kT + tid) * EPV; };
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    const int e0 = id0(it);
    if (vec_ok && e0 + EPV <= s1) {
      q[it] = *reinterpret_cast<const u32x4_t*>(rowp + (size_t)e0 * ESZ);
    } else {
      uint32_t wv[4] = {Tr::fill_word(), Tr::fill_word(), Tr::fill_word(), Tr::fill_word()};
      #pragma unroll 1
      for (int e = 0; e < EPV; ++e) {
        if (e0 + e < s1) {
          const uint32_t r = BF16 ? (uint32_t)(reinterpret_cast<const uint16_t*>(rowp)[e0 + e])
                                  : reinterpret_cast<const uint32_t*>(rowp)[e0 + e];
          const int wi = BF16 ? e >> 1 : e, sh = BF16 ? (e & 1) * 16 : 0;
          const uint32_t msk = BF16 ? (0xFFFFu << sh) : 0xFFFFFFFFu;
          const uint32_t nw = (wv[wi] & ~msk) | (r << sh);
          wv[0] = wi == 0 ? nw : wv[0];
          wv[1] = wi == 1 ? nw : wv[1];
          wv[2] = wi == 2 ? nw : wv[2];
          wv[3] = wi == 3 ? nw : wv[3];
        }
      }
      q[it] = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
    }
  }
}

// Top-K of slice blk, whose vectors are in q.
template <bool BF16, int NV, bool WIDE, int kT, class Smem>
__device__ void scan_block(const ScanArgs& a, Smem& sm, int blk, const u32x4_t (&q)[NV]) {
  using Tr = Traits<BF16>;
  constexpr int kSurvW = 4 * kT;
  constexpr int HCAP = WIDE ? 2 * kT : kHitCap;
  constexpr int SCAP = WIDE ? (BF16 ? kSurvW : kSurvW / 2) : kScanCap;
  constexpr int EPV = Tr::EPV;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int row = blk / a.S, sl = blk - row * a.S;
  const int s0 = sl * a.slice;
  const int s1 = min(a.V, s0 + a.slice);
  const int K = a.K;
  auto id0 = [&](int it) { return s0 + (it * kT + tid) * EPV; };
  // -- largest key per vector and per lane
  uint32_t vk[NV];
  uint32_t lk = 0u;
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    vk[it] = Tr::vec_key_max(q[it]);
    lk = max(lk, vk[it]);
  }
  // -- bound: every active wave vouches for m lanes whose largest key >= its t
  const int nthr_valid = min(kT, (s1 - s0 + EPV - 1) / EPV);
  const int nact = (nthr_valid + kWave - 1) / kWave;
  const int m = nact > 0 ? (K + nact - 1) / nact : K;
  if (nact == 0 && tid == 0) sm.misc[4] = 1;   // empty slice: the exact path yields nothing
  bool block_bound = false;
  {
    // Bound from the whole block: the K-th largest lane maximum, to bin
    // precision (at K = 64 about half the survivors of the per-wave bound
    // below, which remains the fallback). Lane maxima are binned by their
    // key distance below the slice's largest key (bin = one bf16 value, or
    // 2^16 fp32 keys; 255 collects the rest); counting down from the top
    // bin, the first bin b* that brings the count to K gives T, the lowest
    // key bin b* can hold.
    // At least K lanes, hence K elements, reach T (a histogram of the five
    // vector maxima a lane holds gives a tighter T, but its LDS atomics cost
    // more than the smaller survivor set saves). The slice's largest key
    // also bounds the selection's histogram later.
    constexpr int SH = BF16 ? 0 : 16;
    const uint32_t wm = wave_max_u32(lk);
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(&sm.misc[6]), wm);
    __syncthreads();
    const uint32_t hi = (uint32_t)sm.misc[6];
    if (tid < nthr_valid) {
      const uint32_t d = (hi - lk) >> SH;
      atomicAdd(&sm.bhist[d < 255u ? d : 255u], 1);
    }
    __syncthreads();
    if (w == 0) {
      const int b0 = 4 * lane;
      const int h0 = sm.bhist[b0], h1 = sm.bhist[b0 + 1], h2 = sm.bhist[b0 + 2], h3 = sm.bhist[b0 + 3];
      const int sum = h0 + h1 + h2 + h3;
      const int a0 = wave_incl_scan_i32(sum) - sum, a1 = a0 + h0, a2 = a1 + h1, a3 = a2 + h2;
      // misc[7] = b* + 1, left 0 when b* would be the catch-all bin
      if (a0 < K && K <= a1 && b0 < 255) sm.misc[7] = b0 + 1;
      if (a1 < K && K <= a2 && b0 + 1 < 255) sm.misc[7] = b0 + 2;
      if (a2 < K && K <= a3 && b0 + 2 < 255) sm.misc[7] = b0 + 3;
      if (a3 < K && K <= a3 + h3 && b0 + 3 < 255) sm.misc[7] = b0 + 4;
    }
    __syncthreads();
    block_bound = sm.misc[7] > 0 && sm.misc[4] == 0;
  }
  uint32_t T;
  bool bound_ok;
  if (block_bound) {
    const uint32_t hi = (uint32_t)sm.misc[6];
    const uint32_t span = (uint32_t)sm.misc[7] << (BF16 ? 0 : 16);
    T = hi + 1u > span ? hi + 1u - span : 0u;
    bound_ok = true;
  } else {
    // every active wave vouches for m lanes whose largest key >= its t
    if (w < nact) {
      const bool lv = tid < nthr_valid;
      const int nl = __popcll(__ballot(lv));
      if (nl >= m && m <= kWave) {
        const uint32_t t = (WIDE && m > 8) ? wave_mth_largest_sorted(lk, lv, m) : wave_mth_largest(lk, lv, m, Tr::KBITS);
        if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(&sm.misc[2]), ~t);
      } else if (lane == 0) {
        atomicOr(&sm.misc[4], 1);
      }
    }
    __syncthreads();
    bound_ok = sm.misc[4] == 0;
    T = ~(uint32_t)sm.misc[2];
  }
  if (bound_ok) {
    // hit vectors (largest key >= T) go to LDS, one LDS atomic per wave for
    // all its rounds; then one thread per element of a hit vector
    uint64_t bal[NV];
    int nhit = 0;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      bal[it] = __builtin_amdgcn_ballot_w64(vk[it] >= T);
      nhit += __popcll(bal[it]);
    }
    if (nhit) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&sm.misc[5], nhit);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        if (vk[it] >= T) {
          const int hv = base + (int)mbcnt64(bal[it]);
          if (hv < HCAP) {
            sm.hitq[hv] = q[it];
            sm.hitid[hv] = id0(it);
          }
        }
        base += __popcll(bal[it]);
      }
    }
  }
  __syncthreads();
  // wide variant: survivors are counted into the selection's value histogram
  // as they are appended (bins over [T, the slice's largest key])
  const int wshift = hist_shift(T, (uint32_t)sm.misc[6]);
  if constexpr (WIDE) {
   if (bound_ok) {
    // one thread per queued vector, its elements checked in registers; the
    // survivors of a wave are placed by a prefix of the per-thread counts
    // (0..8, four bits, one ballot each) and one LDS atomic
    const int nh = min(sm.misc[5], HCAP);
    for (int v0 = 0; v0 < nh; v0 += kT) {
      const int v = v0 + tid;
      uint32_t smask = 0u, kk[EPV];
      int idb = 0;
      if (v < nh) {
        const u32x4_t qv = sm.hitq[v];
        idb = sm.hitid[v];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          kk[e] = Tr::key(Tr::raw(qv, e));
          smask |= (idb + e < s1 && kk[e] >= T) ? (1u << e) : 0u;
        }
      }
      const uint32_t c = (uint32_t)__popc(smask);
      uint32_t pre = 0u, tot = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint64_t bb = __builtin_amdgcn_ballot_w64((c >> b) & 1u);
        pre += mbcnt64(bb) << b;
        tot += (uint32_t)__popcll(bb) << b;
      }
      int base = 0;
      if (lane == 0 && tot) base = atomicAdd(&sm.misc[3], (int)tot);
      base = __builtin_amdgcn_readfirstlane(base);
      int p = base + (int)pre;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        if ((smask >> e) & 1u) {
          if (p < SCAP) {
            if constexpr (BF16)
              sm.key32[p] = (kk[e] << 16) | (0xFFFFu - (uint32_t)(idb + e - s0));
            else
              sm.key[p] = ((uint64_t)kk[e] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(idb + e));
            atomicAdd(&sm.hist[hist_bin(kk[e], T, wshift)], 1);
          }
          ++p;
        }
      }
    }
   }
  } else if (bound_ok) {
    const int nh = min(sm.misc[5], HCAP);
    // two elements a thread per pass, both read before either is used: one
    // pass covers up to 256 hit vectors
    for (int t0 = tid; t0 < nh * EPV; t0 += 2 * kT) {
      bool sv[2];
      uint32_t kk[2];
      int idx[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = t0 + u * kT;
        const int hv = min(t, nh * EPV - 1) / EPV, e = t - hv * EPV;
        idx[u] = sm.hitid[hv] + e;
        kk[u] = Tr::key(Tr::raw(sm.hitq[hv], e & (EPV - 1)));
        sv[u] = t < nh * EPV && idx[u] < s1 && kk[u] >= T;
      }
      const uint64_t b0 = __builtin_amdgcn_ballot_w64(sv[0]), b1 = __builtin_amdgcn_ballot_w64(sv[1]);
      const int n0 = __popcll(b0), n01 = n0 + __popcll(b1);
      int base = 0;
      if (lane == 0 && n01) base = atomicAdd(&sm.misc[3], n01);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (sv[u]) {
          const int p = base + (u ? n0 : 0) + (int)mbcnt64(u ? b1 : b0);
          if (p < SCAP) {
            if constexpr (BF16)
              sm.key32[p] = (kk[u] << 16) | (0xFFFFu - (uint32_t)(idx[u] - s0));
            else
              sm.key[p] = ((uint64_t)kk[u] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx[u]);
          }
        }
      }
    }
  }
  __syncthreads();
  int ns = sm.misc[3];
  uint32_t lo_v = T;   // every survivor's value key is >= lo_v
  const bool exact = !bound_ok || sm.misc[5] > HCAP || ns > SCAP;
  if (exact) {
    if constexpr (WIDE) {
      for (int i = tid; i < 256; i += kT) sm.hist[i] = 0;
    }
    // -- exact path: Th = K-th largest key (bitwise search on block counts),
    //    then among keys == Th the largest complemented ids (lowest ids)
    int nvalid = 0;
#pragma unroll
    for (int it = 0; it < NV; ++it) nvalid += max(0, min(EPV, s1 - id0(it)));
    const int need = min(K, block_sum(sm, nvalid));
    uint32_t Th = 0;
    for (int b = Tr::KBITS - 1; b >= 0; --b) {
      const uint32_t cand = Th | (1u << b);
      int n = 0;
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e0 = id0(it);
        #pragma unroll 1
        for (int e = 0; e < EPV; ++e) n += (e0 + e < s1 && Tr::key(Tr::raw(q[it], e)) >= cand) ? 1 : 0;
      }
      if (block_sum(sm, n) >= need) Th = cand;
    }
    int ngt = 0;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e0 = id0(it);
      #pragma unroll 1
      for (int e = 0; e < EPV; ++e) ngt += (e0 + e < s1 && Tr::key(Tr::raw(q[it], e)) > Th) ? 1 : 0;
    }
    const int take = need - block_sum(sm, ngt);   // ties at Th to take, lowest ids first
    lo_v = Th;
    uint32_t Ui = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = Ui | (1u << b);
      int n = 0;
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e0 = id0(it);
        #pragma unroll 1
        for (int e = 0; e < EPV; ++e)
          n += (e0 + e < s1 && Tr::key(Tr::raw(q[it], e)) == Th && 0xFFFFFFFFu - (uint32_t)(e0 + e) >= cand) ? 1 : 0;
      }
      if (block_sum(sm, n) >= take) Ui = cand;
    }
    if (tid == 0) sm.misc[3] = 0;
    __syncthreads();
    int c = 0;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e0 = id0(it);
      #pragma unroll 1
      for (int e = 0; e < EPV; ++e) {
        const uint32_t kk = Tr::key(Tr::raw(q[it], e));
        const uint32_t ci = 0xFFFFFFFFu - (uint32_t)(e0 + e);
        c += (e0 + e < s1 && (kk > Th || (kk == Th && ci >= Ui))) ? 1 : 0;
      }
    }
    if (c) {
      int p = atomicAdd(&sm.misc[3], c);
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e0 = id0(it);
        #pragma unroll 1
        for (int e = 0; e < EPV; ++e) {
          const uint32_t kk = Tr::key(Tr::raw(q[it], e));
          const uint32_t ci = 0xFFFFFFFFu - (uint32_t)(e0 + e);
          if (e0 + e < s1 && (kk > Th || (kk == Th && ci >= Ui))) {
            if constexpr (BF16)
              sm.key32[p++] = (kk << 16) | (0xFFFFu - (uint32_t)(e0 + e - s0));
            else
              sm.key[p++] = ((uint64_t)kk << 32) | ci;
          }
        }
      }
    }
    __syncthreads();
    ns = sm.misc[3];
    if constexpr (BF16) {
      // keys of the overflowed pass may remain past ns: the ranking reads up
      // to 7 keys beyond ns and needs zeros there
      if (tid < 32) sm.key32[ns + tid] = 0u;
      __syncthreads();
    }
  }
  if constexpr (WIDE) {
    HistSmem hs{(LDS int*)sm.hist, (LDS int*)sm.cursor, (LDS int*)sm.base, (LDS int*)&sm.misc[0],
                (LDS uint64_t*)sm.bucket, (LDS uint64_t*)sm.out, kSurvW};
    if (!exact) {
      // the histogram is complete: boundary, buckets, ranks
      hist_boundary(K, hs);
      lds_sync();
      const int bstar = sm.misc[0], narea = sm.misc[1];
      for (int i = tid; i < ns; i += kT) {
        uint64_t x;
        uint32_t hv;
        if constexpr (BF16) {
          const uint32_t k32 = sm.key32[i];
          const uint32_t idx = (uint32_t)s0 + 0xFFFFu - (k32 & 0xFFFFu);
          hv = k32 >> 16;
          x = ((uint64_t)hv << 32) | (uint64_t)(0xFFFFFFFFu - idx);
        } else {
          x = sm.key[i];
          hv = (uint32_t)(x >> 32);
        }
        hist_scatter(x, hist_bin(hv, T, wshift), bstar, hs);
      }
      lds_sync();
      hist_rank_out(K, T, wshift, narea, hs);
    } else {
    // survivors, as 64-bit keys, ordered by the value histogram (ns <= the
    // bucket space, so the selection cannot run out of room)
    uint64_t kr[kSurvW / kT];
#pragma unroll
    for (int e = 0; e < kSurvW / kT; ++e) {
      const int i = tid + e * kT;
      uint64_t x = 0ull;
      if (i < ns) {
        if constexpr (BF16) {
          const uint32_t k32 = sm.key32[i];
          const uint32_t idx = (uint32_t)s0 + 0xFFFFu - (k32 & 0xFFFFu);
          x = ((uint64_t)(k32 >> 16) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
        } else {
          x = sm.key[i];
        }
      }
      kr[e] = x;
    }
    lds_sync();   // misc[0..1] and the hit queue's space are reused
    hist_topk<kSurvW / kT>(kr, lo_v, (uint32_t)sm.misc[6], K, hs);
    }
  } else if constexpr (BF16) {
    rank_select32(sm, ns, K, s0);
  } else {
    rank_select(sm, ns, K);
  }
  if (a.S == 1) {
    int32_t* ids = a.cand_ids + (size_t)row * K;
    float* vals = a.cand_logit + (size_t)row * K;
    for (int i = tid; i < K; i += kT) {
      const uint64_t x = sm.out[i];
      ids[i] = x ? (int32_t)(0xFFFFFFFFu - (uint32_t)x) : -1;
      vals[i] = x ? Tr::value((uint32_t)(x >> 32)) : -__builtin_huge_valf();
    }
  } else {
    uint64_t* lst = a.lists + ((size_t)row * a.S + sl) * K;
    for (int i = tid; i < K; i += kT) lst[i] = sm.out[i];
  }
}

template <int G, int kWaves>
__device__ void head_block(const ScanArgs& a, HeadSmem& sm, int tile) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int ntn = a.r / 16;
  const int nt = tile % ntn, mt = tile / ntn;
  const int KS = a.D / 32;
  const int k0 = (KS * w) / kWaves, k1 = (KS * (w + 1)) / kWaves;
  const int m = mt * 16 + (lane & 15);   // this lane's operand row of H
  // rows read coalesced (four adjacent lanes on one 64-byte segment), then
  // permuted to the operand lanes
  const int mc = mt * 16 + coal_row(lane), nc = nt * 16 + coal_row(lane);
  const uint16_t* hrow = a.H + (size_t)(mc < a.M ? mc : 0) * a.D + coal_col(lane);
  const uint16_t* prow = a.Pt + (size_t)nc * a.D + coal_col(lane);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
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
        u16x8_t x = to_mfma_lanes(av[g], lane);
        if (m >= a.M) x = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        acc = mfma_bf16(x, to_mfma_lanes(bv[g], lane), acc);
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

// One tree wave's A fragments as fp16: for tile t (16 rows) and local
// k-step kl of its half of the state, lane l holds row 32 aw + 16 t + (l & 15),
// columns 32 (4 hk + kl) + 8 (l >> 4) .. + 7; stored contiguously per
// (wave, tile, k-step) so the tree kernel reads 1 KB runs.
__device__ void afrag_block(const ScanArgs& a, int tw) {
  const int hk = tw >> 3, aw = tw & 7;
  for (int v = threadIdx.x; v < 2 * 4 * kWave; v += blockDim.x) {
    const int t = v >> 8, kl = (v >> 6) & 3, l = v & 63;
    const int row = aw * 32 + t * 16 + (l & 15), col = (hk * 4 + kl) * 32 + (l >> 4) * 8;
    const u16x8_t x = *reinterpret_cast<const u16x8_t*>(a.A + (size_t)row * 256 + col);
    *reinterpret_cast<h16x8_t*>(a.a_frag + ((size_t)((tw * 2 + t) * 4 + kl) * kWave + l) * 8) = bf16x8_to_f16(x);
  }
}

// One 64 x 64 tile of h[M][r] = H[M][D] * P[D][r] (Pt stored [r][D]) by a
// 1024-thread workgroup on v_mfma_f32_16x16x32_bf16, fragments read from
// LDS. Wave w takes the 32 x 32 quadrant w % 4 (2 x 2 sub-tiles, so each
// fragment it reads feeds two MFMAs) and, of every stage's four k-steps, the
// k-step w / 4; the four partial quadrants are added in LDS in a fixed order
// at the end. Each stage of 128 columns of D is one 16-byte vector of H and
// one of P a thread. Stages are loaded four ahead into a ring of registers
// (slot = stage % 4, the stage loop unrolled by four so that slots and LDS
// buffers are named statically; D is a multiple of 512), and each stage is
// written to the other LDS buffer while the current one feeds the MFMAs.
// Every load is unconditional: past the last stage the last one is read
// again, and rows of H past M read row 0 (an output row depends only on the
// same row of H, and rows past M are not stored). The compiler's wait before a
// stage's LDS write then counts exactly the three younger stages' loads, and
// the per-stage barriers wait for LDS traffic only, so about three stages of
// loads stay in flight.
//
// Workgroups go to the eight XCDs in turn, and head workgroup f lands on XCD
// f mod 8 (both in a head-only launch and when the head tiles are spread one
// in 33 blocks through the stress round's scan grid). Tiles are handed out so
// that each XCD takes one contiguous run of row-major tiles: its L2 then
// fetches a few row blocks of H (and the P blocks) once instead of every row
// block. Any order gives the same results.
__device__ void head_block_big(const ScanArgs& a, HeadBigSmem& sm, int f) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int ntn = a.r / kHB;
  const int tile = a.n_head % 8 == 0 ? (f % 8) * (a.n_head / 8) + f / 8 : f;
  const int nt = tile % ntn, mt = tile / ntn;
  const int m0 = mt * kHB, n0 = nt * kHB;
  const int sr = tid >> 4, sc = (tid & 15) * 8;   // staging: row 0..63, column 0..120
  const uint16_t* ag = a.H + (size_t)(m0 + sr < a.M ? m0 + sr : 0) * a.D + sc;
  const uint16_t* bg = a.Pt + (size_t)(n0 + sr) * a.D + sc;
  const int NS = a.D / kHS;
  u16x8_t pa[4], pb[4];
  auto load = [&](int u, int st) {
    const size_t off = (size_t)(st < NS ? st : NS - 1) * kHS;
    pa[u] = *reinterpret_cast<const u16x8_t*>(ag + off);
    pb[u] = *reinterpret_cast<const u16x8_t*>(bg + off);
  };
  auto stage_to_lds = [&](int u, int buf) {
    *reinterpret_cast<u16x8_t*>(&sm.a[buf][sr][sc]) = pa[u];
    *reinterpret_cast<u16x8_t*>(&sm.b[buf][sr][sc]) = pb[u];
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) load(u, u);
  stage_to_lds(0, 0);
  lds_sync();
  const int qm = (w & 3) >> 1, qn = w & 1, ksl = w >> 2;
  const int fr = lane & 15, kc = ksl * 32 + (lane >> 4) * 8;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int st0 = 0; st0 < NS; st0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cur = u & 1;   // stage st0 + u, st0 a multiple of 4
      load(u, st0 + u + 4);    // slot u held stage st0 + u, already in LDS
      const u16x8_t fa0 = *reinterpret_cast<const u16x8_t*>(&sm.a[cur][qm * 32 + fr][kc]);
      const u16x8_t fa1 = *reinterpret_cast<const u16x8_t*>(&sm.a[cur][qm * 32 + 16 + fr][kc]);
      const u16x8_t fb0 = *reinterpret_cast<const u16x8_t*>(&sm.b[cur][qn * 32 + fr][kc]);
      const u16x8_t fb1 = *reinterpret_cast<const u16x8_t*>(&sm.b[cur][qn * 32 + 16 + fr][kc]);
      acc[0][0] = mfma_bf16(fa0, fb0, acc[0][0]);
      acc[0][1] = mfma_bf16(fa0, fb1, acc[0][1]);
      acc[1][0] = mfma_bf16(fa1, fb0, acc[1][0]);
      acc[1][1] = mfma_bf16(fa1, fb1, acc[1][1]);
      stage_to_lds((u + 1) & 3, cur ^ 1);   // past the last stage: never read
      lds_sync();
    }
  }
  // partial quadrants [k-step][64][64 + 1] over the staging buffers, then
  // each thread adds the four partials of four outputs in k-step order
  LDS float* part = (LDS float*)&sm.a[0][0][0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = qm * 32 + i * 16 + (lane >> 4) * 4 + e, col = qn * 32 + j * 16 + (lane & 15);
        part[(ksl * kHB + row) * (kHB + 1) + col] = acc[i][j][e];
      }
  lds_sync();
#pragma unroll
  for (int q = 0; q < kHB * kHB / 1024; ++q) {
    const int idx = tid + q * 1024, row = idx / kHB, col = idx % kHB;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) v += part[(k * kHB + row) * (kHB + 1) + col];
    if (m0 + row < a.M) a.h[(size_t)(m0 + row) * a.r + n0 + col] = v;
  }
}

__device__ __forceinline__ void clear_words(const ScanArgs& a) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n_clear; i += gridDim.x * blockDim.x) a.clear[i] = 0u;
}

template <bool BF16, int NV>
__global__ __launch_bounds__(kT) void scan_kernel(ScanArgs a) {
  __shared__ KernelSmem smem;
  const int b = blockIdx.x;
  clear_words(a);
  if (b < a.n_scan) {
    if (threadIdx.x < 8) smem.scan.misc[threadIdx.x] = 0;
    if (threadIdx.x < 256) smem.scan.bhist[threadIdx.x] = 0;
    if (BF16)
      for (int i = threadIdx.x; i < kScanCap + 32; i += kT) smem.scan.key32[i] = 0u;
    __syncthreads();
    u32x4_t q[NV];
    load_slice<BF16, NV, kT>(a, b, q);
    scan_block<BF16, NV, false, kT>(a, smem.scan, b, q);
  } else if (b < a.n_scan + a.n_head) {
    head_block<8, kWaves>(a, smem.head, b - a.n_scan);
  } else {
    afrag_block(a, b - a.n_scan - a.n_head);
  }
}

// The same launch for K > 64, with the wide selection: two workgroups fit a
// CU (<= 64 VGPRs, ~60 KB of LDS), so one's selection overlaps the other's
// loads when rows outnumber the CUs. The head tiles are spread evenly over
// the grid (block b is a head tile when floor((b + 1) n_head / total) steps
// up), so their MFMA and cache traffic overlaps the scan's HBM reads
// instead of trailing it.
template <bool BF16, int NV>
__global__ __launch_bounds__(kWideT) __attribute__((amdgpu_waves_per_eu(8))) void scan_wide_kernel(ScanArgs a) {
  __shared__ WideKernelSmem<kWideT> smem;
  const int b = blockIdx.x;
  clear_words(a);
  const int mixed = a.n_scan + a.n_head;
  if (b < mixed) {
    const int f1 = (int)(((long long)(b + 1) * a.n_head) / mixed);
    const int f0 = (int)(((long long)b * a.n_head) / mixed);
    if (f1 == f0) {
      if (threadIdx.x < 8) smem.scan.misc[threadIdx.x] = 0;
      for (int i = threadIdx.x; i < 256; i += kWideT) {
        smem.scan.hist[i] = 0;
        smem.scan.cursor[i] = 0;
        smem.scan.bhist[i] = 0;
      }
      u32x4_t q[NV];
      load_slice<BF16, NV, kWideT>(a, b - f1, q);
      __syncthreads();
      scan_block<BF16, NV, true, kWideT>(a, smem.scan, b - f1, q);
    } else if (a.head_big) {
      head_block_big(a, smem.headbig, f0);
    } else {
      head_block<4, kWideT / kWave>(a, smem.head, f0);
    }
  } else {
    afrag_block(a, b - mixed);
  }
}

// Per-row merge of S sorted slice lists (used when a row spans several slices).
// Every slice holds K keys at or above its K-th, so the row's K-th largest
// value is at least the largest of the slices' K-th values: that value and the
// largest head bound the histogram selection. Massive ties fall back to the
// bound-and-rank selection.
template <int EPT>
__global__ __launch_bounds__(kT) void merge_kernel(const uint64_t* __restrict__ lists, int S, int K, bool bf16,
                                                   int32_t* __restrict__ cand_ids, float* __restrict__ cand_logit) {
  __shared__ uint64_t s_key[kScanCap];
  __shared__ int s_pay[kScanCap];
  __shared__ uint64_t s_out[1024];
  __shared__ int s_outp[1024];
  __shared__ int s_misc[8];
  __shared__ int s_hist[256], s_cursor[256], s_base[256], s_hmisc[2];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (tid < 8) s_misc[tid] = 0;
  for (int i = tid; i < 256; i += kT) {
    s_hist[i] = 0;
    s_cursor[i] = 0;
  }
  __syncthreads();
  const uint64_t* L = lists + (size_t)row * S * K;
  uint32_t lo_v = 0u, hi_v = 0u;
  for (int sl = 0; sl < S; ++sl) {
    hi_v = max(hi_v, (uint32_t)(L[(size_t)sl * K] >> 32));
    lo_v = max(lo_v, (uint32_t)(L[(size_t)sl * K + K - 1] >> 32));
  }
  uint64_t k[EPT];
  int p[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid + e * kT;
    k[e] = i < S * K ? L[i] : 0ull;
    p[e] = 0;
  }
  HistSmem hs{(LDS int*)s_hist, (LDS int*)s_cursor, (LDS int*)s_base, (LDS int*)s_hmisc, (LDS uint64_t*)s_key,
              (LDS uint64_t*)s_out, kScanCap};
  if (!hist_topk<EPT>(k, lo_v, hi_v, K, hs)) {
    SelSmem sm{(LDS uint64_t*)s_key, (LDS int*)s_pay, (LDS uint64_t*)s_out, (LDS int*)s_outp,
               (LDS int*)s_misc, kScanCap};
    block_select<EPT>(k, p, K, bf16 ? 16 : 32, sm);
  }
  for (int i = tid; i < K; i += kT) {
    const uint64_t x = s_out[i];
    cand_ids[(size_t)row * K + i] = x ? (int32_t)(0xFFFFFFFFu - (uint32_t)x) : -1;
    cand_logit[(size_t)row * K + i] =
        x ? (bf16 ? bf16_key_to_f32((uint32_t)(x >> 32)) : key_to_f32((uint32_t)(x >> 32))) : -__builtin_huge_valf();
  }
}

// The same merge by pairs of lists, for up to eight lists: the lists (padded
// with empty ones to a power of two) are merged pairwise, level by level, in
// LDS. Keys are distinct and nonzero (0 marks an empty slot), so a key's place
// in the merge of its list a with the partner list b is its index in a plus
// the number of b's keys above it (a binary search in the descending list b);
// places at or past K are dropped. log2(lists) levels of one search per key,
// against the value histogram's dozen barriers. Same output, key for key.
constexpr int kMergeSortedMaxS = 8;
#ifndef DARTREE_MERGE_NT
#define DARTREE_MERGE_NT 1024
#endif
constexpr int kMergeT = DARTREE_MERGE_NT;
__global__ __launch_bounds__(kMergeT) void merge_sorted_kernel(const uint64_t* __restrict__ lists, int S, int K,
                                                               bool bf16, int32_t* __restrict__ cand_ids,
                                                               float* __restrict__ cand_logit) {
  extern __shared__ __align__(16) char smem_raw[];
  int P = 1;
  while (P < S) P <<= 1;
  LDS uint64_t* buf0 = (LDS uint64_t*)smem_raw;
  LDS uint64_t* buf1 = buf0 + (size_t)P * K;
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint64_t* Lr = lists + (size_t)row * S * K;
  for (int i = tid; i < P * K; i += kMergeT) buf0[i] = i < S * K ? Lr[i] : 0ull;
  __syncthreads();
  LDS uint64_t* cur = buf0;
  LDS uint64_t* nxt = buf1;
  for (int n = P; n > 1; n >>= 1) {
    for (int i = tid; i < (n >> 1) * K; i += kMergeT) nxt[i] = 0ull;
    __syncthreads();
    for (int i = tid; i < n * K; i += kMergeT) {
      const uint64_t x = cur[i];
      if (x == 0ull) continue;
      const int l = i / K, j = i - l * K;
      const LDS uint64_t* b = cur + (size_t)(l ^ 1) * K;
      int lo = 0, hi = K;   // first place in b whose key is below x = b's keys above x
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (b[mid] > x) lo = mid + 1;
        else hi = mid;
      }
      const int r = j + lo;
      if (r < K) nxt[(size_t)(l >> 1) * K + r] = x;
    }
    __syncthreads();
    LDS uint64_t* t = cur;
    cur = nxt;
    nxt = t;
  }
  for (int i = tid; i < K; i += kMergeT) {
    const uint64_t x = cur[i];
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

}  // namespace

ScanPlan scan_plan(int rows, int V, int K, bool bf16) {
  ScanPlan p{};
  const int epv = bf16 ? 8 : 4;
  // slices per row: as few as keep every thread at <= kMaxNV vectors
  p.wide = K > 64;
  const int nt = p.wide ? kWideT : kT;
  const long long per_wg = (long long)nt * epv * kMaxNV;
  p.S = (int)((V + per_wg - 1) / per_wg);
  long long sl = ((long long)V + p.S - 1) / p.S;
  sl = (sl + epv - 1) / epv * epv;   // slice length: multiple of the vector width
  p.slice = (int)sl;
  const int nvec = (int)((sl + epv - 1) / epv);
  p.nv = (nvec + nt - 1) / nt;
  p.n_scan = rows * p.S;
  p.merge_ept = (p.S * K + kT - 1) / kT <= 8 ? 8 : 16;
  p.list_bytes = p.S > 1 ? (size_t)rows * p.S * K * sizeof(uint64_t) : 0;
  p.ok = p.nv >= 1 && p.nv <= kMaxNV && (long long)p.S * K <= 16LL * kT;
  return p;
}

bool head_mfma_ok(bool bf16, const void* H, const void* Pt, int D, int r) {
  return bf16 && D % 32 == 0 && r % 16 == 0 && ((((uintptr_t)H) | ((uintptr_t)Pt)) & 15u) == 0;
}

bool head_big_ok(int M, int D, int r) { return M >= kHB && r % kHB == 0 && D % (4 * kHS) == 0; }

int head_tiles(bool big, int M, int r) {
  return big ? (r / kHB) * ((M + kHB - 1) / kHB) : (r / 16) * ((M + 15) / 16);
}

hipError_t launch_scan(const ScanPlan& p, bool bf16, const ScanArgs& args_in, hipStream_t s) {
  ScanArgs a = args_in;
  a.S = p.S;
  a.slice = p.slice;
  a.n_scan = p.n_scan;
  const int grid = a.n_scan + a.n_head + a.n_afrag;
  if (grid == 0) return hipSuccess;
#define DT_SCAN(B, NVV)                                                                  \
  do {                                                                                    \
    if (p.wide)                                                                           \
      hipLaunchKernelGGL((scan_wide_kernel<B, NVV>), dim3(grid), dim3(kWideT), 0, s, a);  \
    else                                                                                  \
      hipLaunchKernelGGL((scan_kernel<B, NVV>), dim3(grid), dim3(kT), 0, s, a);           \
  } while (0)
  switch (p.nv) {
    case 1: if (bf16) DT_SCAN(true, 1); else DT_SCAN(false, 1); break;
    case 2: if (bf16) DT_SCAN(true, 2); else DT_SCAN(false, 2); break;
    case 3: if (bf16) DT_SCAN(true, 3); else DT_SCAN(false, 3); break;
    case 4: if (bf16) DT_SCAN(true, 4); else DT_SCAN(false, 4); break;
    default: if (bf16) DT_SCAN(true, 5); else DT_SCAN(false, 5); break;
  }
#undef DT_SCAN
  return hipGetLastError();
}

hipError_t launch_merge(const ScanPlan& p, int rows, int K, bool bf16, const uint64_t* lists, int32_t* cand_ids,
                        float* cand_logit, hipStream_t s) {
  if (p.S <= 1) return hipSuccess;
  if (p.S <= kMergeSortedMaxS) {
    int P = 1;
    while (P < p.S) P <<= 1;
    const size_t lds = (size_t)2 * P * K * sizeof(uint64_t);
    if (lds <= 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)merge_sorted_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(merge_sorted_kernel, dim3(rows), dim3(kMergeT), lds, s, lists, p.S, K, bf16, cand_ids,
                         cand_logit);
      return hipGetLastError();
    }
  }
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
  a.n_scan = 0;
  a.head_big = head_big_ok(M, D, r) ? 1 : 0;
  a.n_head = head_tiles(a.head_big, M, r);
  if (a.head_big)
    hipLaunchKernelGGL((scan_wide_kernel<true, 1>), dim3(a.n_head), dim3(kWideT), 0, s, a);
  else
    hipLaunchKernelGGL((scan_kernel<true, 1>), dim3(a.n_head), dim3(kT), 0, s, a);
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
