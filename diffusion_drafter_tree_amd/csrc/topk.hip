// Step a1: per-position top-K candidates from the base logits in one HBM pass.
//
// DARTree (marsggbo blog, section 3.1, candidate generation): every block
// position keeps its K best tokens of the drafter's base logits; everything
// else can never become a tree node. The order is value descending, then
// token id ascending.
//
// Layout: logits[rows][V] (bf16 bits or fp32), rows = n_req * L. A row is cut
// into chunks of CE elements; one 1024-thread workgroup per (row, chunk)
// streams its chunk with 16-byte loads, keeps the chunk's exact top-K as
// 64-bit keys (value key << 32 | ~id), and the last workgroup of each row to
// finish (atomic ticket) merges the per-chunk lists. A row with one chunk is
// finished by its only workgroup.
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkCap = 4096;

template <bool BF16>
__device__ __forceinline__ uint64_t make_key(uint32_t raw, uint32_t idx) {
  uint32_t k = BF16 ? bf16_key(raw) : f32_key(__uint_as_float(raw));
  return ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

template <bool BF16>
__device__ __forceinline__ void write_candidate(uint64_t sk, int32_t* ids, float* vals, int i) {
  if (sk == 0ull) {
    ids[i] = -1;
    vals[i] = -__builtin_huge_valf();
    return;
  }
  uint32_t k = (uint32_t)(sk >> 32);
  ids[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)sk);
  vals[i] = BF16 ? bf16_key_to_f32(k) : key_to_f32(k);
}

template <bool BF16, int NV, int EPTM>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const void* __restrict__ logits, int V, int K, int C,
                                                           uint64_t* __restrict__ lists,
                                                           unsigned int* __restrict__ tickets,
                                                           int32_t* __restrict__ cand_ids,
                                                           float* __restrict__ cand_logit) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ESZ;            // elements per 16-byte vector
  constexpr int EPT = NV * EPV;            // keys per thread in the chunk pass
  constexpr int CE = kTopkThreads * EPT;   // elements per chunk
  __shared__ uint64_t s_buf[kTopkCap];
  __shared__ uint64_t s_out[1024];
  __shared__ int s_rank[kRankMax];
  __shared__ int s_misc[8];
  TopkSmem sm{s_buf, s_out, s_rank, s_misc, kTopkCap};

  const int tid = threadIdx.x;
  const int row = blockIdx.x / C;
  const int ch = blockIdx.x - row * C;
  const int c0 = ch * CE;
  const int c1 = min(V, c0 + CE);
  const char* rowp = static_cast<const char*>(logits) + (size_t)row * (size_t)V * ESZ;
  const bool aligned = ((uintptr_t)rowp & 15u) == 0;

  uint64_t sk[EPT];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e0 = c0 + v * (kTopkThreads * EPV) + tid * EPV;
    if (aligned && e0 + EPV <= c1) {
      u32x4_t q = *reinterpret_cast<const u32x4_t*>(rowp + (size_t)e0 * ESZ);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        uint32_t raw = BF16 ? ((q[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) : q[e];
        sk[v * EPV + e] = make_key<BF16>(raw, (uint32_t)(e0 + e));
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int idx = e0 + e;
        uint64_t key = 0ull;
        if (idx < c1) {
          uint32_t raw = BF16 ? (uint32_t)(reinterpret_cast<const uint16_t*>(rowp)[idx])
                              : reinterpret_cast<const uint32_t*>(rowp)[idx];
          key = make_key<BF16>(raw, (uint32_t)idx);
        }
        sk[v * EPV + e] = key;
      }
    }
  }
  const int n = block_topk<EPT>(sk, K, sm);
  (void)n;
  if (C == 1) {
    for (int i = tid; i < K; i += kTopkThreads)
      write_candidate<BF16>(s_out[i], cand_ids + (size_t)row * K, cand_logit + (size_t)row * K, i);
    return;
  }
  uint64_t* mine = lists + ((size_t)row * C + ch) * K;
  for (int i = tid; i < K; i += kTopkThreads) mine[i] = s_out[i];
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    unsigned int old = atomicAdd(&tickets[row], 1u);
    s_misc[7] = (old == (unsigned int)(C - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_misc[7]) return;
  __threadfence();
  const uint64_t* all = lists + (size_t)row * C * K;
  const int total = C * K;
  uint64_t mk[EPTM];
#pragma unroll
  for (int e = 0; e < EPTM; ++e) {
    const int i = tid + e * kTopkThreads;
    mk[e] = i < total ? all[i] : 0ull;
  }
  block_topk<EPTM>(mk, K, sm);
  for (int i = tid; i < K; i += kTopkThreads)
    write_candidate<BF16>(s_out[i], cand_ids + (size_t)row * K, cand_logit + (size_t)row * K, i);
  if (tid == 0) tickets[row] = 0u;
}

}  // namespace

TopkPlan topk_plan(int rows, int V, int K, bool bf16) {
  TopkPlan p{};
  const int epv = bf16 ? 8 : 4;
  // vectors per thread: the smallest that keeps the per-row merge within 16
  // keys per thread (and at most 16 keys per thread in the chunk pass)
  int nv_options[2] = {bf16 ? 1 : 2, bf16 ? 2 : 4};
  p.nv = 0;
  for (int o = 0; o < 2; ++o) {
    int nv = nv_options[o];
    int ce = kTopkThreads * nv * epv;
    int c = (V + ce - 1) / ce;
    if (c == 1 || (long long)c * K <= 16LL * kTopkThreads) {
      p.nv = nv;
      p.chunks = c;
      p.chunk_elems = ce;
      break;
    }
  }
  if (p.nv == 0) return p;
  p.merge_ept = (p.chunks == 1 || (long long)p.chunks * K <= 8LL * kTopkThreads) ? 8 : 16;
  p.grid = rows * p.chunks;
  p.list_bytes = p.chunks > 1 ? (size_t)rows * p.chunks * K * sizeof(uint64_t) : 0;
  p.ticket_bytes = (size_t)rows * sizeof(unsigned int);
  return p;
}

hipError_t launch_topk(const TopkPlan& p, bool bf16, const void* logits, int V, int K, uint64_t* lists,
                       unsigned int* tickets, int32_t* cand_ids, float* cand_logit, hipStream_t s) {
  dim3 grid(p.grid), block(kTopkThreads);
#define DT_TOPK(B, NVV, EM) \
  hipLaunchKernelGGL((topk_kernel<B, NVV, EM>), grid, block, 0, s, logits, V, K, p.chunks, lists, tickets, cand_ids, \
                     cand_logit)
  if (bf16) {
    if (p.nv == 1) { if (p.merge_ept == 8) DT_TOPK(true, 1, 8); else DT_TOPK(true, 1, 16); }
    else { if (p.merge_ept == 8) DT_TOPK(true, 2, 8); else DT_TOPK(true, 2, 16); }
  } else {
    if (p.nv == 2) { if (p.merge_ept == 8) DT_TOPK(false, 2, 8); else DT_TOPK(false, 2, 16); }
    else { if (p.merge_ept == 8) DT_TOPK(false, 4, 8); else DT_TOPK(false, 4, 16); }
  }
#undef DT_TOPK
  return hipGetLastError();
}

}  // namespace dartree
