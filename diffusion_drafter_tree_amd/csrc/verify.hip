// Verification consumer of the emitted draft tree, with a synthetic target.
//
// DARTree (marsggbo blog, section 3.2): the drafted tree is verified by the
// target in one forward pass under a tree-attention mask, and the longest
// root path the target agrees with is accepted. Here the target is synthetic:
// per request a continuation target[0..L-1] (the target's token at depth d is
// target[d - 1]), and one attention head over the draft nodes stands in for the
// target's layers:
//   acceptance  a node is accepted iff its token equals the target's at its
//               depth and its parent is the anchor or accepted; tau = 1 + the
//               depth of the deepest accepted node (the target's own next
//               token counts), and the accepted path's nodes are listed;
//   attention   out[i] = sum_j softmax_j(<Q[i], K[j]> / sqrt(dh)) V[j] over
//               the nodes j whose bit is set in mask row i (the node and its
//               ancestors); rows past n_sel are zero.
// Up to four 1024-thread workgroups per request. In workgroup 0 a thread per
// node walks its root path for the acceptance. A wave per query row (rows
// round-robin over all the request's waves) iterates over the set bits of its
// mask row with a running (online) softmax, its lanes over the head
// dimension, each dot product added across the wave in a fixed order. The
// request's token, depth and parent arrays and its target are read into LDS
// once (the walks are chains of dependent reads), and so are its K and V rows
// when they fit (kVerifyKVBytes), so that a query's ancestors are LDS reads.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kVT = 1024;
constexpr int kMaxDh = 256;
constexpr int kMaxTreeB = 1024;                  // the library's largest B
constexpr size_t kVerifyKVBytes = 96 * 1024;     // K and V rows staged up to this size

__global__ __launch_bounds__(kVT) void verify_kernel(VerifyArgs a, int kv_staged) {
  __shared__ int s_best;
  __shared__ int s_tok[kMaxTreeB], s_dep[kMaxTreeB], s_par[kMaxTreeB], s_tgt[32];
  extern __shared__ float s_kv[];   // [2][B][dh] when kv_staged
  // blockIdx.y = g of G workgroups a request: workgroup 0 also does the
  // acceptance; the query rows go round-robin over the G * 16 waves
  const int q = blockIdx.x, g = blockIdx.y, G = gridDim.y, tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int L = a.L, B = a.B, dh = a.dh;
  const int n = min(max(a.n_sel[q], 0), B);
  for (int i = tid; i < B; i += kVT) {
    s_tok[i] = a.tok[(size_t)q * B + i];
    s_dep[i] = a.depth[(size_t)q * B + i];
    s_par[i] = a.parent[(size_t)q * B + i];
  }
  if (tid < L) s_tgt[tid] = a.target[(size_t)q * L + tid];
  if (kv_staged) {
    const float* kg = a.K + (size_t)q * B * dh;
    const float* vg = a.V + (size_t)q * B * dh;
    for (int i = tid; i < B * dh; i += kVT) {
      s_kv[i] = kg[i];
      s_kv[(size_t)B * dh + i] = vg[i];
    }
  }
  const int32_t* tok = s_tok;
  const int32_t* dep = s_dep;
  const int32_t* par = s_par;
  const int32_t* tgt = s_tgt;
  if (tid == 0) s_best = -1;
  __syncthreads();
  // ---- acceptance: deepest node whose whole root path matches the target
  for (int i = tid; i < (g == 0 ? n : 0); i += kVT) {
    const int d = dep[i];
    bool ok = d >= 1 && d <= L;
    int v = i, steps = 0;
    while (ok && v >= 0 && steps <= L) {
      const int dv = dep[v];
      ok = dv >= 1 && dv <= L && tok[v] == tgt[dv - 1];
      const int pv = par[v];
      v = pv >= 0 && pv < v ? pv : -1;
      ++steps;
    }
    if (ok) atomicMax(&s_best, (d << 16) | i);
  }
  __syncthreads();
  if (g == 0 && tid == 0) {
    const int b = s_best;
    const int dbest = b < 0 ? 0 : b >> 16;
    a.acc_len[q] = 1 + dbest;
    int32_t* nodes = a.acc_nodes + (size_t)q * L;
    for (int d = dbest; d < L; ++d) nodes[d] = -1;
    int v = b < 0 ? -1 : (b & 0xFFFF);
    for (int d = dbest; d >= 1 && v >= 0; --d) {
      nodes[d - 1] = v;
      const int pv = par[v];
      v = pv >= 0 && pv < v ? pv : -1;
    }
  }
  // ---- one attention step under the tree mask, a wave per query row
  const int words = (B + 63) / 64;
  const float scale = 1.0f / sqrtf((float)dh);
  constexpr int PL = kMaxDh / kWave;   // head-dimension elements per lane
  for (int i = g * (kVT / kWave) + w; i < B; i += G * (kVT / kWave)) {
    float* orow = a.out + ((size_t)q * B + i) * dh;
    if (i >= n) {
      for (int e = lane; e < dh; e += kWave) orow[e] = 0.f;
      continue;
    }
    const float* qrow = a.Q + ((size_t)q * B + i) * dh;
    float qv[PL], acc[PL];
#pragma unroll
    for (int t = 0; t < PL; ++t) {
      const int e = lane + t * kWave;
      qv[t] = e < dh ? qrow[e] : 0.f;
      acc[t] = 0.f;
    }
    float m = -__builtin_huge_valf(), l = 0.f;
    const uint64_t* mrow = a.mask + ((size_t)q * B + i) * words;
    for (int wi = 0; wi < words; ++wi) {
      uint64_t bits = mrow[wi];
      while (bits) {
        const int j = wi * 64 + __builtin_ctzll(bits);
        bits &= bits - 1;
        if (j >= B) break;
        const float* krow = kv_staged ? s_kv + (size_t)j * dh : a.K + ((size_t)q * B + j) * dh;
        const float* vrow = kv_staged ? s_kv + ((size_t)B + j) * dh : a.V + ((size_t)q * B + j) * dh;
        float part = 0.f, vv[PL];
#pragma unroll
        for (int t = 0; t < PL; ++t) {
          const int e = lane + t * kWave;
          part = e < dh ? fmaf(qv[t], krow[e], part) : part;
          vv[t] = e < dh ? vrow[e] : 0.f;
        }
        const float s = wave_sum_f32(part) * scale;
        const float mn = fmaxf(m, s);
        const float c = expf(m - mn), p = expf(s - mn);
        l = l * c + p;
#pragma unroll
        for (int t = 0; t < PL; ++t) acc[t] = fmaf(acc[t], c, p * vv[t]);
        m = mn;
      }
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int t = 0; t < PL; ++t) {
      const int e = lane + t * kWave;
      if (e < dh) orow[e] = acc[t] * inv;
    }
  }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
  const size_t kv = 2ull * a.B * a.dh * sizeof(float);
  const int staged = kv <= kVerifyKVBytes ? 1 : 0;
  const size_t smem = staged ? kv : 0;
  if (smem > 0) {
    const hipError_t e = hipFuncSetAttribute((const void*)verify_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)smem);
    if (e != hipSuccess) return e;
  }
  // up to four workgroups a request, each with at least one query row a wave
  const int G = std::max(1, std::min(4, (a.B + kVT / kWave - 1) / (kVT / kWave)));
  hipLaunchKernelGGL(verify_kernel, dim3(a.n_req, G), dim3(kVT), smem, s, a, staged);
  return hipGetLastError();
}

}  // namespace dartree
