// Steps a2 + a3: depth-by-depth batched correction scoring, the score
// s_beta, per-depth top-W pruning and the survivors' head states.
//
// DARTree (marsggbo blog, section 3.1): at depth d every surviving parent of
// depth d-1 goes through the correction head in one batched call and scores
// its children; a child's score is s_beta(u_1..u_d) = sum_i log q_i(u_i) +
// beta * d with beta <= 0; each depth keeps its top W (the fixed-width
// supertree). AINews summary: one batched head call per depth replaces one
// call per node. The head is the declared low-rank stand-in:
//   z[p][c]  = Lbase_d[c] + <s_p, U[c]>,   log q = log-softmax over the K
//              candidates of depth d (clamped to <= 0 so that a child never
//              outscores its parent in fp32);
//   s_child  = tanh(A s_p + E[u] + h_d)     (only needed when d < L).
//
// One 1024-thread workgroup per request runs the dependent depth loop. Its
// states, scores and selection live in LDS. On the bf16-weight path both
// contractions (S U_C^T and A S^T) run on v_mfma_f32_16x16x32_bf16 with each
// fp32 state split exactly into three bf16 parts, so every product is exact
// and only the fp32 accumulation rounds. The fp32-weight path uses fp32 FMAs.
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kExpThreads = 1024;
constexpr int kExpWaves = kExpThreads / kWave;
constexpr int kExpCap = 2048;
constexpr int kExpEPT = 8;   // children per thread: W * K <= 8192

__device__ __forceinline__ float ldw(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldw(const float* p, size_t i) { return p[i]; }

struct ExpSmem {
  float* S;       // [W][r]   states of the current parents
  float* AS;      // [W][r]   A * s_p
  float* Z;       // [W][K]   corrected logits, then cum
  float* cumP;    // [W]
  float* lse;     // [W]
  int* cid;       // [K]
  float* clog;    // [K]
  int* lv_tok;    // [W]
  int* lv_ps;     // [W]
  float* lv_cum;  // [W]
  float* lv_sb;   // [W]
  uint64_t* buf;  // [kExpCap]
  uint64_t* out;  // [W]
  int* rank;      // [kRankMax]
  int* misc;      // [8]
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline size_t exp_layout(int K, int W, int r, ExpSmem* sm, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align16(off + bytes);
    return o;
  };
  size_t oS = take(sizeof(float) * W * r);
  size_t oAS = take(sizeof(float) * W * r);
  size_t oZ = take(sizeof(float) * W * K);
  size_t ocP = take(sizeof(float) * W);
  size_t olse = take(sizeof(float) * W);
  size_t ocid = take(sizeof(int) * K);
  size_t oclog = take(sizeof(float) * K);
  size_t otok = take(sizeof(int) * W);
  size_t ops = take(sizeof(int) * W);
  size_t ocum = take(sizeof(float) * W);
  size_t osb = take(sizeof(float) * W);
  size_t obuf = take(sizeof(uint64_t) * kExpCap);
  size_t oout = take(sizeof(uint64_t) * W);
  size_t orank = take(sizeof(int) * kRankMax);
  size_t omisc = take(sizeof(int) * 8);
  if (sm) {
    sm->S = (float*)(base + oS);
    sm->AS = (float*)(base + oAS);
    sm->Z = (float*)(base + oZ);
    sm->cumP = (float*)(base + ocP);
    sm->lse = (float*)(base + olse);
    sm->cid = (int*)(base + ocid);
    sm->clog = (float*)(base + oclog);
    sm->lv_tok = (int*)(base + otok);
    sm->lv_ps = (int*)(base + ops);
    sm->lv_cum = (float*)(base + ocum);
    sm->lv_sb = (float*)(base + osb);
    sm->buf = (uint64_t*)(base + obuf);
    sm->out = (uint64_t*)(base + oout);
    sm->rank = (int*)(base + orank);
    sm->misc = (int*)(base + omisc);
  }
  return off;
}

// Z[p][k] = clog[k] + <S[p], U[cid[k]]>, bf16 U on MFMA with the 3-way split.
__device__ void score_mfma(const ExpSmem& sm, const uint16_t* __restrict__ U, int Wp, int K, int r) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int MT = (Wp + 15) / 16, NT = (K + 15) / 16, KS = r / 32;
  const int sub = (lane >> 4) * 8;
  for (int t = w; t < MT * NT; t += kExpWaves) {
    const int mt = t / NT, nt = t - mt * NT;
    const int p = mt * 16 + (lane & 15);
    const int k = nt * 16 + (lane & 15);
    const bool pv = p < Wp, kv = k < K;
    const uint16_t* urow = U + (size_t)(kv ? sm.cid[k] : 0) * r;
    const float* srow = sm.S + (size_t)(pv ? p : 0) * r;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
      const int j0 = ks * 32 + sub;
      u16x8_t b = *reinterpret_cast<const u16x8_t*>(urow + j0);
      if (!kv) b = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      u16x8_t ah, am, al;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t h, m, l;
        split3(pv ? srow[j0 + i] : 0.f, h, m, l);
        ah[i] = (unsigned short)h;
        am[i] = (unsigned short)m;
        al[i] = (unsigned short)l;
      }
      acc = mfma_bf16(al, b, acc);
      acc = mfma_bf16(am, b, acc);
      acc = mfma_bf16(ah, b, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = mt * 16 + (lane >> 4) * 4 + i;
      if (pp < Wp && kv) sm.Z[pp * K + k] = acc[i] + sm.clog[k];
    }
  }
}

// AS[p][j] = sum_m A[j][m] S[p][m], bf16 A on MFMA with the 3-way split.
__device__ void state_mfma(const ExpSmem& sm, const uint16_t* __restrict__ A, int Wp, int r) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int MT = r / 16, NT = (Wp + 15) / 16, KS = r / 32;
  const int sub = (lane >> 4) * 8;
  for (int t = w; t < MT * NT; t += kExpWaves) {
    const int mt = t / NT, nt = t - mt * NT;
    const int j = mt * 16 + (lane & 15);
    const int p = nt * 16 + (lane & 15);
    const bool pv = p < Wp;
    const uint16_t* arow = A + (size_t)j * r;
    const float* srow = sm.S + (size_t)(pv ? p : 0) * r;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
      const int m0 = ks * 32 + sub;
      u16x8_t a = *reinterpret_cast<const u16x8_t*>(arow + m0);
      u16x8_t bh, bm, bl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t h, m, l;
        split3(pv ? srow[m0 + i] : 0.f, h, m, l);
        bh[i] = (unsigned short)h;
        bm[i] = (unsigned short)m;
        bl[i] = (unsigned short)l;
      }
      acc = mfma_bf16(a, bl, acc);
      acc = mfma_bf16(a, bm, acc);
      acc = mfma_bf16(a, bh, acc);
    }
    if (pv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.AS[p * r + mt * 16 + (lane >> 4) * 4 + i] = acc[i];
    }
  }
}

template <typename WT>
__device__ void score_valu(const ExpSmem& sm, const WT* __restrict__ U, int Wp, int K, int r) {
  for (int idx = threadIdx.x; idx < Wp * K; idx += kExpThreads) {
    const int p = idx / K, k = idx - p * K;
    const size_t ub = (size_t)sm.cid[k] * r;
    const float* srow = sm.S + (size_t)p * r;
    float acc = 0.f;
    for (int j = 0; j < r; ++j) acc = fmaf(srow[j], ldw(U, ub + j), acc);
    sm.Z[idx] = acc + sm.clog[k];
  }
}

template <typename WT>
__device__ void state_valu(const ExpSmem& sm, const WT* __restrict__ A, int Wp, int r) {
  for (int idx = threadIdx.x; idx < Wp * r; idx += kExpThreads) {
    const int p = idx / r, j = idx - p * r;
    const float* srow = sm.S + (size_t)p * r;
    float acc = 0.f;
    for (int m = 0; m < r; ++m) acc = fmaf(ldw(A, (size_t)j * r + m), srow[m], acc);
    sm.AS[idx] = acc;
  }
}

template <typename WT, bool MF>
__global__ __launch_bounds__(kExpThreads) void expand_kernel(ExpandArgs a) {
  extern __shared__ __align__(16) char smem_raw[];
  ExpSmem sm;
  exp_layout(a.K, a.W, a.r, &sm, smem_raw);
  const int q = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int L = a.L, K = a.K, W = a.W, r = a.r;
  const WT* A = static_cast<const WT*>(a.A);
  const WT* E = static_cast<const WT*>(a.E);
  const WT* U = static_cast<const WT*>(a.U);
  const float* hq = a.h + (size_t)q * L * r;
  int32_t* st_tok = a.st_tok + (size_t)q * L * W;
  int32_t* st_ps = a.st_parent + (size_t)q * L * W;
  float* st_cum = a.st_cum + (size_t)q * L * W;
  float* st_sb = a.st_sbeta + (size_t)q * L * W;
  int32_t* st_cnt = a.st_count + (size_t)q * L;
  float* st_state = a.st_state + (size_t)q * W * r;

  // parents of depth d0: the root (state h_0, cum 0) or the stored level d0-1
  int Wp;
  if (a.d0 == 1) {
    Wp = 1;
    for (int j = tid; j < r; j += kExpThreads) sm.S[j] = hq[j];
    if (tid == 0) sm.cumP[0] = 0.f;
  } else {
    Wp = st_cnt[a.d0 - 2];
    Wp = Wp < 1 ? 1 : (Wp > W ? W : Wp);
    for (int i = tid; i < Wp * r; i += kExpThreads) sm.S[i] = st_state[i];
    for (int i = tid; i < Wp; i += kExpThreads) sm.cumP[i] = st_cum[(size_t)(a.d0 - 2) * W + i];
  }
  TopkSmem tsm{sm.buf, sm.out, sm.rank, sm.misc, kExpCap};

  for (int d = a.d0; d <= a.d1; ++d) {
    // candidates of depth d (ids clamped into [0, V) so a bad id cannot fault)
    const int32_t* cid_g = a.cand_ids + ((size_t)q * L + (d - 1)) * K;
    const float* clog_g = a.cand_logit + ((size_t)q * L + (d - 1)) * K;
    for (int k = tid; k < K; k += kExpThreads) {
      int c = cid_g[k];
      sm.cid[k] = (c < 0 || c >= a.V) ? 0 : c;
      sm.clog[k] = clog_g[k];
    }
    __syncthreads();
    const bool need_state = d < L;
    if (MF) {
      score_mfma(sm, reinterpret_cast<const uint16_t*>(U), Wp, K, r);
      if (need_state) state_mfma(sm, reinterpret_cast<const uint16_t*>(A), Wp, r);
    } else {
      score_valu<WT>(sm, U, Wp, K, r);
      if (need_state) state_valu<WT>(sm, A, Wp, r);
    }
    __syncthreads();
    // log-softmax over the K candidates of each parent; Z becomes cum
    for (int p = w; p < Wp; p += kExpWaves) {
      float* zr = sm.Z + (size_t)p * K;
      float m = -__builtin_huge_valf();
      for (int k = lane; k < K; k += kWave) m = fmaxf(m, zr[k]);
      m = wave_max_f32(m);
      float s = 0.f;
      for (int k = lane; k < K; k += kWave) s += expf(zr[k] - m);
      s = wave_sum_f32(s);
      const float lse = m + logf(s);
      const float cp = sm.cumP[p];
      for (int k = lane; k < K; k += kWave) zr[k] = cp + fminf(zr[k] - lse, 0.f);
    }
    __syncthreads();
    // keys of all children: s_beta desc, token asc, parent slot asc
    const float bd = a.beta * (float)d;
    const int nchild = Wp * K;
    uint64_t keys[kExpEPT];
#pragma unroll
    for (int e = 0; e < kExpEPT; ++e) {
      const int i = tid + e * kExpThreads;
      uint64_t key = 0ull;
      if (i < nchild) {
        const int p = i / K, k = i - p * K;
        const float sb = sm.Z[i] + bd;
        const uint32_t lo = 0xFFFFFFFFu - (((uint32_t)sm.cid[k] << 9) | (uint32_t)p);
        key = ((uint64_t)f32_key(sb) << 32) | lo;
      }
      keys[e] = key;
    }
    const int nk = block_topk<kExpEPT>(keys, W, tsm);
    // each thread finds its own children among the kept keys
    const uint64_t last = sm.out[nk - 1];
#pragma unroll
    for (int e = 0; e < kExpEPT; ++e) {
      if (keys[e] != 0ull && keys[e] >= last) {
        int lo = 0, hi = nk - 1;
        while (lo < hi) {   // out[] is strictly descending
          const int mid = (lo + hi) >> 1;
          if (sm.out[mid] > keys[e]) lo = mid + 1; else hi = mid;
        }
        const int i = tid + e * kExpThreads;
        const int p = i / K, k = i - p * K;
        sm.lv_tok[lo] = sm.cid[k];
        sm.lv_ps[lo] = p;
        sm.lv_cum[lo] = sm.Z[i];
        sm.lv_sb[lo] = sm.Z[i] + bd;
      }
    }
    __syncthreads();
    for (int s = tid; s < W; s += kExpThreads) {
      const size_t o = (size_t)(d - 1) * W + s;
      const bool v = s < nk;
      st_tok[o] = v ? sm.lv_tok[s] : -1;
      st_ps[o] = v ? sm.lv_ps[s] : -1;
      st_cum[o] = v ? sm.lv_cum[s] : -__builtin_huge_valf();
      st_sb[o] = v ? sm.lv_sb[s] : -__builtin_huge_valf();
    }
    if (tid == 0) st_cnt[d - 1] = nk;
    if (need_state) {
      const float* hd = hq + (size_t)d * r;
      for (int i = tid; i < nk * r; i += kExpThreads) {
        const int s = i / r, j = i - s * r;
        const float x = (sm.AS[(size_t)sm.lv_ps[s] * r + j] + ldw(E, (size_t)sm.lv_tok[s] * r + j)) + hd[j];
        sm.S[i] = tanhf(x);
      }
      for (int s = tid; s < nk; s += kExpThreads) sm.cumP[s] = sm.lv_cum[s];
    }
    Wp = nk;
    __syncthreads();
  }
  if (a.d1 < L) {
    for (int i = tid; i < Wp * r; i += kExpThreads) st_state[i] = sm.S[i];
  }
}

}  // namespace

size_t expand_smem_bytes(int K, int W, int r) { return exp_layout(K, W, r, nullptr, nullptr); }

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s) {
  const size_t smem = expand_smem_bytes(a.K, a.W, a.r);
  const bool mf = a.bf16 && (a.r % 32 == 0) && (((uintptr_t)a.U | (uintptr_t)a.A) & 15u) == 0;
  dim3 grid(a.n_req), block(kExpThreads);
  hipError_t e = hipSuccess;
#define DT_EXP(T, M)                                                                                       \
  do {                                                                                                     \
    e = hipFuncSetAttribute((const void*)expand_kernel<T, M>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                            (int)smem);                                                                    \
    if (e != hipSuccess) return e;                                                                         \
    hipLaunchKernelGGL((expand_kernel<T, M>), grid, block, smem, s, a);                                    \
  } while (0)
  if (a.bf16) {
    if (mf) DT_EXP(uint16_t, true); else DT_EXP(uint16_t, false);
  } else {
    DT_EXP(float, false);
  }
#undef DT_EXP
  return hipGetLastError();
}

}  // namespace dartree
