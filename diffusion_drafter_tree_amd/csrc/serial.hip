// Heap-serial draft-tree construction ("pop then correct"), the baseline the
// deferred round is measured against.
//
// DARTree (marsggbo blog, section 2 and section 4.3, Table 2): a best-first
// tree builder pops the best pending node, runs the correction head on it and
// pushes its children, one node at a time, so every node costs a dependent
// head call; the deferred construction batches a whole depth per call
// instead. Here, per request and with the same stand-in head as the round:
//   the root's state is h_0 and its K children (the candidates of depth 1)
//   are pending; B times: pop the best pending node by the round's comparator
//   (s_beta descending, depth ascending, token ascending, then the parent's
//   own order, which is its pop index because nodes are popped in comparator
//   order); when its depth d < L, compute its state tanh(A s_parent + E[u] +
//   h_d) and push all K candidates of depth d + 1 with
//   cum = cum_parent + min(log-softmax of Lbase + <s, U[c]>, 0) and
//   s_beta = cum + beta (d + 1). No per-depth width applies.
//
// One 1024-thread workgroup per request. Pending nodes live in LDS; after each
// push only the best (B - pops) of them are kept, since no other can be popped
// within the budget. Node states go to a workspace, [n][B + 1][r] fp32 (slot 0
// the root, slot i the i-th popped node). Weights are bf16 or fp32, arithmetic
// fp32 FMAs; tanh, exp and log from the device library.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kT = 1024;
constexpr int kPoolCap = kSerialMaxB + 1024;   // pending nodes kept + one push of K
constexpr int kCandStage = 4096;               // L * K candidates staged in LDS

__device__ __forceinline__ float ldw(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldw(const float* p, size_t i) { return p[i]; }

// out[i] = <M[row_i], vec> for i < nrows (row_i = rows[i], clamped into
// [0, nv), or i when rows is NULL): a wave takes RPW rows at a time, its
// lanes read 16-byte vectors along the rows (all RPW rows' loads issued
// before their FMAs, kept as raw vectors until then), and each row's partial
// sums are added across the wave in a fixed order. All threads of the
// workgroup call it; the caller syncs.
template <typename WT, int RPW = 8>
__device__ __forceinline__ void rows_dot(const WT* __restrict__ M, const int32_t* __restrict__ rows, int nrows,
                                         int nv, int r, const float* vec, float* out) {
  constexpr int EPL = 16 / (int)sizeof(WT);   // elements per 16-byte load
  using V16 = std::conditional_t<sizeof(WT) == 2, u16x8_t, f32x4_t>;
  const int lane = lane_id(), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const bool vec_ok = r % EPL == 0 && (((uintptr_t)M) & 15u) == 0;
  for (int i0 = w * RPW; i0 < nrows; i0 += nw * RPW) {
    float acc[RPW];
    const WT* base[RPW];
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      acc[u] = 0.f;
      const int i = min(i0 + u, nrows - 1);
      int row = rows ? rows[i] : i;
      row = row < 0 || row >= nv ? 0 : row;
      base[u] = M + (size_t)row * r;
    }
    for (int c0 = lane * EPL; c0 < r; c0 += kWave * EPL) {
      if (vec_ok) {
        V16 raw[RPW];
#pragma unroll
        for (int u = 0; u < RPW; ++u) raw[u] = *reinterpret_cast<const V16*>(base[u] + c0);
#pragma unroll
        for (int u = 0; u < RPW; ++u) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            float x;
            if constexpr (sizeof(WT) == 2) x = bf16_to_f32((uint32_t)raw[u][e]);
            else x = raw[u][e];
            acc[u] = fmaf(x, vec[c0 + e], acc[u]);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < RPW; ++u)
          for (int e = 0; e < EPL && c0 + e < r; ++e) acc[u] = fmaf(ldw(base[u], (size_t)(c0 + e)), vec[c0 + e], acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const float t = wave_sum_f32(acc[u]);
      if (lane == 0 && i0 + u < nrows) out[i0 + u] = t;
    }
  }
}

struct SerialSmem {
  uint64_t key[kPoolCap];
  float cum[kPoolCap];
  int tok[kPoolCap];
  int dep[kPoolCap];   // depth << 16 | parent pop index (0 = root)
  int rank[kPoolCap];
  float s_par[1024];   // the popped node's parent state
  float s_new[1024];   // the popped node's state
  float part[1024];    // A s_parent
  float z[1024];       // corrected logits of the children
  int c_id[kCandStage];    // every depth's candidate ids and base logits, when
  float c_lg[kCandStage];  // L * K fits (read once instead of once a pop)
  unsigned long long best;
  int misc[8];
};

template <typename WT>
__global__ __launch_bounds__(kT) void serial_kernel(SerialArgs a) {
  __shared__ SerialSmem sm;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int q = blockIdx.x;
  const int L = a.L, K = a.K, B = a.B, r = a.r;
  const WT* A = static_cast<const WT*>(a.A);
  const WT* E = static_cast<const WT*>(a.E);
  const WT* U = static_cast<const WT*>(a.U);
  const float* hq = a.h + (size_t)q * L * r;
  float* st = a.states + (size_t)q * (B + 1) * r;
  int32_t* o_tok = a.tok + (size_t)q * B;
  int32_t* o_dep = a.depth + (size_t)q * B;
  int32_t* o_par = a.parent + (size_t)q * B;
  float* o_sc = a.score + (size_t)q * B;

  // the root: state h_0, cum 0
  for (int j = tid; j < r; j += kT) {
    st[j] = hq[j];
    sm.s_new[j] = hq[j];
  }
  // The pending count lives in a register of every thread: push, prune and
  // pop change it the same way everywhere, so it needs no LDS round trip and
  // no barrier guards it.
  int npend = 0;
  const bool staged = L * K <= kCandStage;
  if (staged) {
    const int32_t* cg = a.cand_ids + (size_t)q * L * K;
    const float* lg = a.cand_logit + (size_t)q * L * K;
    for (int i = tid; i < L * K; i += kT) {
      sm.c_id[i] = cg[i];
      sm.c_lg[i] = lg[i];
    }
  }
  __syncthreads();

  // Scores the K children (depth d) of the node in sm.s_new with cumulative
  // score cum_p and pop index pidx, and appends them to the pending pool.
  auto push_children = [&](int d, float cum_p, int pidx) {
    const int32_t* C = staged ? sm.c_id + (size_t)(d - 1) * K : a.cand_ids + ((size_t)q * L + d - 1) * K;
    const float* base = staged ? sm.c_lg + (size_t)(d - 1) * K : a.cand_logit + ((size_t)q * L + d - 1) * K;
    rows_dot<WT>(U, C, K, a.V, r, sm.s_new, sm.z);
    __syncthreads();
    // one wave: the base logits added, the log-softmax over the K, the keys
    // appended (each lane keeps its own k's, so no barrier in between)
    if (w == 0) {
      float m = -__builtin_huge_valf();
      for (int k = lane; k < K; k += kWave) {
        const float z = sm.z[k] + base[k];
        sm.z[k] = z;
        m = fmaxf(m, z);
      }
      m = wave_max_f32(m);
      float ssum = 0.f;
      for (int k = lane; k < K; k += kWave) ssum += expf(sm.z[k] - m);
      ssum = wave_sum_f32(ssum);
      const float lse = m + logf(ssum);
      const int n0 = npend;
      for (int k = lane; k < K; k += kWave) {
        const float cum = cum_p + fminf(sm.z[k] - lse, 0.f);
        const float sb = cum + a.beta * (float)d;
        const uint32_t tk = (uint32_t)C[k] & 0x3FFFFu;
        const uint32_t lo = ((uint32_t)d << 27) | (tk << 9) | (uint32_t)pidx;
        sm.key[n0 + k] = ((uint64_t)f32_key(sb) << 32) | (uint64_t)(0xFFFFFFFFu - lo);
        sm.cum[n0 + k] = cum;
        sm.tok[n0 + k] = C[k];
        sm.dep[n0 + k] = (d << 16) | pidx;
      }
    }
    npend += K;
    __syncthreads();
  };

  // Keeps the best `keep` pending nodes (distinct keys; ranks by counting).
  auto prune = [&](int keep) {
    const int n = npend;
    if (n <= keep) return;
    for (int i = tid; i < n; i += kT) {
      const uint64_t x = sm.key[i];
      int rk = 0;
      for (int j = 0; j < n; ++j) rk += sm.key[j] > x ? 1 : 0;
      sm.rank[i] = rk;
    }
    __syncthreads();
    // stable compaction in rank order: entry of rank t moves to slot t
    uint64_t kx[2];
    float cx[2];
    int tx[2], dx[2], rx[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * kT;
      rx[u] = i < n ? sm.rank[i] : keep;
      if (i < n) {
        kx[u] = sm.key[i];
        cx[u] = sm.cum[i];
        tx[u] = sm.tok[i];
        dx[u] = sm.dep[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (rx[u] < keep) {
        sm.key[rx[u]] = kx[u];
        sm.cum[rx[u]] = cx[u];
        sm.tok[rx[u]] = tx[u];
        sm.dep[rx[u]] = dx[u];
      }
    }
    npend = keep;
    __syncthreads();
  };

  push_children(1, 0.f, 0);
  prune(B);
  int npop = 0;
  for (int i = 0; i < B; ++i) {
    // every thread has read the pending count of the last push or prune (a
    // prune may return without a barrier) before wave 0 changes it below
    __syncthreads();
    const int n = npend;
    if (n == 0) break;
    // pop, by one wave: the largest key (keys are distinct and nonzero, so
    // the maximum and its slot are unique), its outputs, and its removal (the
    // last pending node takes its place); the popped node's fields go to
    // misc[2..5] for the workgroup
    if (w == 0) {
      unsigned long long lb = 0ull;
      int lj = -1;
      for (int j = lane; j < n; j += kWave) {
        const unsigned long long kj = sm.key[j];
        if (kj > lb) {
          lb = kj;
          lj = j;
        }
      }
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t ohi = (uint32_t)__shfl_xor((int)(uint32_t)(lb >> 32), o);
        const uint32_t olo = (uint32_t)__shfl_xor((int)(uint32_t)lb, o);
        const int oj = __shfl_xor(lj, o);
        const unsigned long long ok = ((unsigned long long)ohi << 32) | olo;
        if (ok > lb) {
          lb = ok;
          lj = oj;
        }
      }
      if (lane == 0) {
        const int jb = lb != 0ull ? lj : -1;
        sm.misc[2] = jb;
        if (jb >= 0) {
          const int tk = sm.tok[jb], dp = sm.dep[jb];
          sm.misc[3] = tk;
          sm.misc[4] = dp;
          sm.misc[5] = __float_as_int(sm.cum[jb]);
          o_tok[i] = tk;
          o_dep[i] = dp >> 16;
          o_par[i] = (dp & 0xFFFF) - 1;
          o_sc[i] = key_to_f32((uint32_t)(lb >> 32));
          const int last = n - 1;
          sm.key[jb] = sm.key[last];
          sm.cum[jb] = sm.cum[last];
          sm.tok[jb] = sm.tok[last];
          sm.dep[jb] = sm.dep[last];
        }
      }
    }
    __syncthreads();
    const int jb = sm.misc[2];
    if (jb < 0) break;   // cannot happen while n > 0; leaves the remaining slots padded
    npend = n - 1;
    const float cum = __int_as_float(sm.misc[5]);
    const int tk = sm.misc[3], d = sm.misc[4] >> 16, pidx = sm.misc[4] & 0xFFFF;
    npop = i + 1;
    if (d < L) {
      // its state from its parent's (workspace slot pidx)
      // (r <= 1024 = kT: thread j owns element j; its E and h elements are
      // loaded with the parent state, ahead of the A product)
      const float* sp = st + (size_t)pidx * r;
      const float* hd = hq + (size_t)d * r;
      const WT* erow = E + (size_t)(tk < 0 || tk >= a.V ? 0 : tk) * r;
      float ev = 0.f, hv = 0.f;
      if (tid < r) {
        sm.s_par[tid] = sp[tid];
        ev = ldw(erow, (size_t)tid);
        hv = hd[tid];
      }
      __syncthreads();
      if (A != nullptr) rows_dot<WT>(A, nullptr, r, r, r, sm.s_par, sm.part);   // no A: the Markov head
      __syncthreads();
      if (tid < r) {
        const float v = tanhf((A != nullptr ? sm.part[tid] : 0.f) + ev + hv);
        sm.s_new[tid] = v;
        st[(size_t)(i + 1) * r + tid] = v;
      }
      __syncthreads();
      push_children(d + 1, cum, i + 1);
    }
    prune(B - i - 1);
  }
  for (int i = npop + tid; i < B; i += kT) {
    o_tok[i] = -1;
    o_dep[i] = 0;
    o_par[i] = -2;
    o_sc[i] = -__builtin_huge_valf();
  }
  if (tid == 0) a.n_sel[q] = npop;
}

}  // namespace

hipError_t launch_serial(const SerialArgs& a, bool bf16w, hipStream_t s) {
  if (bf16w)
    hipLaunchKernelGGL((serial_kernel<uint16_t>), dim3(a.n_req), dim3(kT), 0, s, a);
  else
    hipLaunchKernelGGL((serial_kernel<float>), dim3(a.n_req), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace dartree
