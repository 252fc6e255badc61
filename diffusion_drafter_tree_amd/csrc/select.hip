// Steps a4 + a5: deferred global top-B over the supertree, breadth-first
// emission with parent pointers, and the tree-attention ancestor bitmask.
//
// DARTree (marsggbo blog, section 3.1, deferred pruning): after the supertree
// is built, the B best nodes are chosen in one pass; Lemma 1 states that for
// beta <= 0 this set is prefix-closed and equals best-first heap pops on the
// materialised tree. Section 3.2: the target verifies every path at once under
// a tree-attention mask. Order of the emitted nodes: depth, then the parent's
// emitted index, then token id. Mask row i has bit j set iff j == i or node j
// is an ancestor of i (bit j % 64 of word j / 64).
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelCap = 2048;   // >= L * W (L <= 31, W <= 64)

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ uint64_t s_buf[kSelCap];
  __shared__ uint64_t s_out[1024];
  __shared__ int s_rank[kRankMax];
  __shared__ int s_misc[8];
  __shared__ int s_cnt[32];
  __shared__ int s_ps[kSelCap];
  __shared__ int s_tok[kSelCap];
  __shared__ float s_sb[kSelCap];
  __shared__ int s_emit[kSelCap];   // emitted index, or -1 when not selected
  __shared__ int s_k2[64];
  __shared__ int s_nd[32];          // selected nodes per depth
  TopkSmem tsm{s_buf, s_out, s_rank, s_misc, kSelCap};
  const int q = blockIdx.x, tid = threadIdx.x;
  const int L = a.L, W = a.W, B = a.B;
  const int32_t* cnt_g = a.st_count + (size_t)q * L;
  const size_t lw = (size_t)q * L * W;
  for (int d = tid; d < 32; d += kSelThreads) {
    s_cnt[d] = d < L ? min(max(cnt_g[d], 0), W) : 0;
    s_nd[d] = 0;
  }
  __syncthreads();
  uint64_t keys[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = tid + e * kSelThreads;
    uint64_t key = 0ull;
    if (i < L * W) {
      const int d = i / W + 1, s = i - (d - 1) * W;
      if (s < s_cnt[d - 1]) {
        const int tok = a.st_tok[lw + i];
        int ps = a.st_parent[lw + i];
        ps = d == 1 ? 0 : ps;
        const float sb = a.st_sbeta[lw + i];
        s_ps[i] = ps;
        s_tok[i] = tok;
        s_sb[i] = sb;
        const uint32_t lo = 0xFFFFFFFFu - (((uint32_t)d << 27) | (((uint32_t)tok & 0x3FFFFu) << 9) | ((uint32_t)ps & 0x1FFu));
        key = ((uint64_t)f32_key(sb) << 32) | lo;
      }
    }
    keys[e] = key;
  }
  const int n = block_topk<2>(keys, B, tsm);
  const uint64_t last = n > 0 ? s_out[n - 1] : ~0ull;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = tid + e * kSelThreads;
    if (i < L * W) {
      const bool sel = keys[e] != 0ull && keys[e] >= last;
      s_emit[i] = sel ? 0 : -1;
      if (sel) atomicAdd(&s_nd[i / W], 1);
    }
  }
  __syncthreads();
  // breadth-first emission, one depth at a time
  int base = 0;
  int32_t* o_tok = a.tok + (size_t)q * B;
  int32_t* o_dep = a.depth + (size_t)q * B;
  int32_t* o_par = a.parent + (size_t)q * B;
  float* o_sc = a.score + (size_t)q * B;
  int32_t* o_slot = a.slot + (size_t)q * B;
  for (int d = 1; d <= L; ++d) {
    const int nd = s_nd[d - 1];
    if (nd == 0) break;   // prefix closure: nothing deeper is selected
    const int c = s_cnt[d - 1];
    const int row = (d - 1) * W;
    int pe = -1, k2 = 0x7FFFFFFF;
    const bool act = tid < c && s_emit[row + tid] >= 0;
    if (act) {
      const int ps = s_ps[row + tid];
      pe = d == 1 ? -1 : s_emit[row - W + min(max(ps, 0), W - 1)];
      k2 = ((pe + 1) << 18) | (s_tok[row + tid] & 0x3FFFF);
    }
    if (tid < 64) s_k2[tid] = (tid < c) ? k2 : 0x7FFFFFFF;
    __syncthreads();
    if (act) {
      int rnk = 0;
      for (int s2 = 0; s2 < c; ++s2) rnk += s_k2[s2] < k2;
      const int e = base + rnk;
      s_emit[row + tid] = e;
      if (e < B) {
        o_tok[e] = s_tok[row + tid];
        o_dep[e] = d;
        o_par[e] = pe;
        o_sc[e] = s_sb[row + tid];
        o_slot[e] = tid;
      }
    }
    base += nd;
    __syncthreads();
  }
  for (int i = n + tid; i < B; i += kSelThreads) {
    o_tok[i] = -1;
    o_dep[i] = 0;
    o_par[i] = -2;
    o_sc[i] = -__builtin_huge_valf();
    o_slot[i] = -1;
  }
  if (tid == 0) a.n_sel[q] = n;
}

// One thread per (row, word): walk the ancestor chain of the row's node and
// collect the bits that fall into that word. The walk follows only pointers
// with -1 <= parent[j] < j and stops after B steps, so any input terminates.
__global__ __launch_bounds__(256) void mask_kernel(int B, const int32_t* __restrict__ n_sel,
                                                   const int32_t* __restrict__ parent, uint64_t* __restrict__ mask) {
  extern __shared__ int s_par[];
  const int q = blockIdx.y;
  const int words = (B + 63) / 64;
  const int32_t* pq = parent + (size_t)q * B;
  for (int i = threadIdx.x; i < B; i += blockDim.x) s_par[i] = pq[i];
  __syncthreads();
  const int ns = min(max(n_sel[q], 0), B);
  const size_t total = (size_t)B * words;
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
    const int i = (int)(t / words), wd = (int)(t % words);
    uint64_t bits = 0ull;
    if (i < ns) {
      int j = i;
      for (int step = 0; step <= B && j >= 0; ++step) {
        if ((j >> 6) == wd) bits |= 1ull << (j & 63);
        const int p = s_par[j];
        if (p >= j || p < -1) break;
        j = p;
      }
    }
    mask[(size_t)q * total + t] = bits;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.n_req), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mask(int n_req, int B, const int32_t* n_sel, const int32_t* parent, uint64_t* mask,
                       hipStream_t s) {
  const int words = (B + 63) / 64;
  const int per_req = B * words;
  const int gx = (per_req + 255) / 256;
  hipLaunchKernelGGL(mask_kernel, dim3(gx, n_req), dim3(256), sizeof(int) * B, s, B, n_sel, parent, mask);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, size_t n_words, uint32_t value, hipStream_t s) {
  if (n_words == 0) return hipSuccess;
  size_t g = (n_words + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)g), dim3(256), 0, s, static_cast<uint32_t*>(p), n_words, value);
  return hipGetLastError();
}

}  // namespace dartree
