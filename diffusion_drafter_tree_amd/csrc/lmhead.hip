// The drafter's LM head fused with the top-K of its logits: candidates taken
// straight from the block's hidden states, the logits never written out.
//
// DARTree (marsggbo blog, section 3.1, basic flow): one block-parallel forward
// of the diffusion drafter gives the block's base logits, and each position's
// K best tokens are the candidates the tree is built from. Here the base
// logits are logits[i][v] = sum_j X[i][j] * Wlm[v][j] for the block's final
// hidden states X [rows][D] and a synthetic head Wlm [V][D], both bf16.
//
// Launch 1 (lmhead_topk_kernel), grid S x ceil(rows / 16): workgroup (s, g)
// owns rows 16g..16g+15 and slab s of the vocabulary (consecutive 16-column
// tiles, ntiles * s / S .. ntiles * (s + 1) / S). Eight waves; wave w takes
// the slab's tiles w, w + 8, ... Per D chunk staged in LDS (the 16 hidden rows,
// bf16), each wave streams its tiles' head rows through a register ring of
// k-steps (16 bytes a lane a step, four adjacent lanes on one 64-byte segment
// of a head row, permuted to the operand lanes; loads issued RING steps ahead) into
// v_mfma_f32_16x16x32_bf16 (products of bf16 are exact, fp32 accumulation)
// and adds each finished tile into the slab's logits in LDS. Then one wave per
// row selects the row's K best logits of the slab exactly: the K-th largest
// 32-bit order key by a bit search over ballot counts, the keys above it and
// the lowest columns among those equal to it, sorted by a 64-lane network, and
// writes them as a sorted list of (value key << 32 | ~id).
// Launch 2 (lmhead_merge_kernel): the S lists of each row merged into its K
// candidates (value descending, id ascending) by bitonic list merges.
//
// The head's HBM stream is the whole cost: V * D * 2 bytes (778 MB at
// V = 151936, D = 2560) against 2 * rows * V * D flops (12.4 GFLOP at 16
// rows), 16 flop a byte, far below the bf16 MFMA ridge. The slab lists are
// rows * S * K * 8 bytes (2 MiB at 16 rows, S = 256, K = 64).
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kLT = 512;                // threads a workgroup
constexpr int kLW = kLT / kWave;        // 8 waves
constexpr int kTPW = 8;                 // tiles a wave may own: a slab has <= 64 tiles
constexpr int kSlabTiles = kLW * kTPW;  // 64 tiles, 1024 columns
constexpr int kMaxSlabs = 256;          // slabs a row: 16 lists a merge wave
constexpr size_t kLdsMax = 160 * 1024;

struct LmArgs {
  const uint16_t* X;   // [rows][D]
  const uint16_t* W;   // [V][D]
  int rows, V, D, K, S, ntiles, kc, slab_cols;
  uint64_t* lists;     // [rows][S][K]
};

template <int RING>
__global__ __launch_bounds__(kLT) void lmhead_topk_kernel(LmArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int s = blockIdx.x, r0 = blockIdx.y * 16;
  const int nr = min(16, a.rows - r0);
  const int t0 = (int)((int64_t)s * a.ntiles / a.S), t1 = (int)((int64_t)(s + 1) * a.ntiles / a.S);
  const int nt = t1 - t0;
  const int col0 = t0 * 16;
  const int ncol = min(t1 * 16, a.V) - col0;
  const int XSTR = a.kc + 8;           // bf16 elements; rows 16 bytes apart in bank terms
  const int LSTR = a.slab_cols + 4;    // floats
  LDS uint16_t* Xs = (LDS uint16_t*)smem;
  LDS float* lg = (LDS float*)(smem + (size_t)16 * XSTR * 2);
  LDS uint64_t* sel = (LDS uint64_t*)(smem + (size_t)16 * XSTR * 2 + (size_t)16 * LSTR * 4);

  for (int i = tid; i < 16 * LSTR; i += kLT) lg[i] = 0.f;

  const int my_nt = nt > w ? (nt - w + kLW - 1) / kLW : 0;
  const int m16 = lane & 15, sub = (lane >> 4) * 8;

  for (int c0 = 0; c0 < a.D; c0 += a.kc) {
    const int kc = min(a.kc, a.D - c0);   // a multiple of 32 * RING
    // every wave is done with the previous chunk (and lg is cleared) before
    // the hidden rows of this chunk are staged
    __syncthreads();
    const int vpr = kc / 8;   // 16-byte vectors a row
    for (int i = tid; i < 16 * vpr; i += kLT) {
      const int r = i / vpr, c = (i - r * vpr) * 8;
      u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < nr) v = *reinterpret_cast<const u16x8_t*>(a.X + (size_t)(r0 + r) * a.D + c0 + c);
      *reinterpret_cast<LDS u16x8_t*>(Xs + r * XSTR + c) = v;
    }
    __syncthreads();

    // The wave's work in this chunk: its tiles j = 0..my_nt-1, each nks
    // k-steps of 32, taken in groups of RING k-steps (nks is a multiple of
    // RING). Two register rings alternate: while one group's MFMAs read one
    // ring, the next group's loads are in flight into the other, issued at the
    // start of the group. Past the last group the loads repeat the last group
    // (every load is issued, so the compiler's wait for a ring counts exactly
    // the RING younger loads of the other one).
    const int nks = kc / 32;
    const int gpt = nks / RING;          // groups a tile
    const int ngroups = my_nt * gpt;
    if (ngroups > 0) {
      // head rows read with four adjacent lanes on one 64-byte segment, then
      // permuted to the MFMA operand lanes (coal_row / to_mfma_lanes)
      auto load_group = [&](u16x8_t (&r)[RING], int g) {
        g = min(g, ngroups - 1);
        const int j = g / gpt, kg = g - j * gpt;
        const int col = min(col0 + (w + j * kLW) * 16 + coal_row(lane), a.V - 1);
        const u16x8_t* src =
            reinterpret_cast<const u16x8_t*>(a.W + (size_t)col * a.D + c0 + kg * RING * 32 + coal_col(lane));
#pragma unroll
        for (int u = 0; u < RING; ++u) r[u] = src[u * 4];
      };
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      auto mma_group = [&](const u16x8_t (&r)[RING], int g) {
        const int j = g / gpt, kg = g - j * gpt;
        const LDS uint16_t* xs = Xs + m16 * XSTR + kg * RING * 32 + sub;
#pragma unroll
        for (int u = 0; u < RING; ++u) {
          const u16x8_t xa = *reinterpret_cast<const LDS u16x8_t*>(xs + u * 32);
          acc = mfma_bf16(xa, to_mfma_lanes(r[u], lane), acc);
        }
        if (kg == gpt - 1) {
          // tile j done for this chunk: rows 4 (lane / 16) + e, column m16
          LDS float* dst = lg + (4 * (lane >> 4)) * LSTR + (w + j * kLW) * 16 + m16;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e * LSTR] += acc[e];
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      };
      u16x8_t ra[RING], rb[RING];
      load_group(ra, 0);
      for (int g = 0; g < ngroups; g += 2) {
        load_group(rb, g + 1);
        mma_group(ra, g);
        load_group(ra, g + 2);
        if (g + 1 < ngroups) mma_group(rb, g + 1);
      }
    }
  }
  __syncthreads();

  // ---- the slab's K best of each row: one wave a row --------------------------
  constexpr int NJ = kSlabTiles * 16 / kWave;   // 16 keys a lane at most
  LDS uint64_t* sw = sel + w * kWave;
  for (int r = w; r < nr; r += kLW) {
    const LDS float* rowp = lg + r * LSTR;
    uint32_t vk[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int c = lane + jj * kWave;
      vk[jj] = c < ncol ? f32_key(rowp[c]) : 0u;   // 0: no column (finite logits never map to 0)
    }
    const int nj = (ncol + kWave - 1) / kWave;
    // T = the K-th largest key of the slab (0 when the slab holds <= K
    // columns): the largest t with at least K keys >= t, bit by bit
    uint32_t T = 0u;
    if (ncol > a.K) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          if (jj < nj) cnt += __popcll(__ballot(vk[jj] >= t));
        if (cnt >= a.K) T = t;
      }
    }
    int gt = 0;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      if (jj < nj) gt += __popcll(__ballot(vk[jj] > T));
    const int need_eq = a.K - gt;   // keys equal to T taken, lowest columns first
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      if (jj < nj) {
        const bool eq = T != 0u && vk[jj] == T;
        const uint64_t be = __ballot(eq);
        const bool take = vk[jj] > T || (eq && eq_seen + (int)mbcnt64(be) < need_eq);
        const uint64_t bt = __ballot(take);
        if (take) {
          const uint32_t id = (uint32_t)(col0 + lane + jj * kWave);
          sw[base + (int)mbcnt64(bt)] = ((uint64_t)vk[jj] << 32) | (uint64_t)(0xFFFFFFFFu - id);
        }
        base += __popcll(bt);
        eq_seen += __popcll(be);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t key = lane < base ? sw[lane] : 0ull;
    uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
    wave_sort_desc(hi, lo);
    if (lane < a.K)
      a.lists[((size_t)(r0 + r) * a.S + s) * a.K + lane] = ((uint64_t)hi << 32) | lo;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

// The S sorted lists of each row (K <= 64 keys each, descending, zero
// padded) merged into the row's K best, one workgroup a row; wave w holds
// lists w, w + 16, ... (16 at most), all loaded at once.
//
// Pruned path: T, the K-th largest value word (the key's high 32 bits) among
// the S list maxima, is reached by K distinct keys, so the row's K-th best
// key has a value word >= T and so has every key of the result. Only the keys
// whose value word is >= T (about K of them when the row's best keys are
// spread over many slabs) are gathered into LDS and ranked by counting. When more than kSurvCap keys reach T (ties across slabs, a head
// whose logits repeat), the lists are merged in full instead: pairwise in a
// tree per wave (the elementwise maximum of one descending list and the other
// reversed holds the K best of both as a bitonic sequence, which six
// half-cleaner stages sort descending), then the 16 waves' results by wave
// 0 the same way. Keys are distinct (each carries its column), so both paths
// give the same K keys in the same order.
constexpr int kMT = 1024, kMW = kMT / kWave;
constexpr int kMPer = kMaxSlabs / kMW;   // lists a wave
constexpr int kSurvCap = kMT;            // survivors the pruned path ranks (one a thread)
static_assert(kMPer == 16, "the merge tree below takes 16 lists a wave");

// K best of 16 sorted lists, one a register pair per lane; the result in
// (h[0], l[0]).
__device__ __forceinline__ void merge_tree16(uint32_t (&h)[16], uint32_t (&l)[16]) {
#pragma unroll
  for (int st = 1; st < 16; st *= 2)
#pragma unroll
    for (int i = 0; i < 16; i += 2 * st) wave_merge_desc(h[i], l[i], ((uint64_t)h[i + st] << 32) | l[i + st]);
}

__global__ __launch_bounds__(kMT) void lmhead_merge_kernel(const uint64_t* __restrict__ lists, int S, int K,
                                                           int32_t* __restrict__ cand_ids,
                                                           float* __restrict__ cand_logit) {
  __shared__ __align__(16) uint32_t mx[kMaxSlabs];   // value words of the list maxima (zero: absent list)
  __shared__ uint64_t sv[kSurvCap];                     // keys whose value word is >= T
  __shared__ uint64_t part[kMW][kWave];                 // full merge: the waves' results
  __shared__ uint32_t thr;
  __shared__ int nsv;
  const int row = blockIdx.x, tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const uint64_t* L = lists + (size_t)row * S * K;
  const bool v = lane < K;
  // addresses clamped into the row's lists (every load is issued), the
  // slots past S and the lanes past K zeroed after
  const int ln = min(lane, K - 1);
  uint64_t kk[kMPer];
#pragma unroll
  for (int i = 0; i < kMPer; ++i) kk[i] = L[(size_t)min(w + i * kMW, S - 1) * K + ln];
  if (tid == 0) {
    thr = 0u;
    nsv = 0;
  }
  uint32_t h[kMPer], l[kMPer];
#pragma unroll
  for (int i = 0; i < kMPer; ++i) {
    const uint64_t x = (v && w + i * kMW < S) ? kk[i] : 0ull;
    h[i] = (uint32_t)(x >> 32);
    l[i] = (uint32_t)x;
    if (lane == 0) mx[w + i * kMW] = h[i];
  }
  __syncthreads();
  {
    // T: the value word m of a maximum with fewer than K maxima above it and
    // at least K at or above it (one value, possibly held by several
    // maxima); four threads a maximum, each counting over a quarter. With
    // fewer than K non-zero maxima it is zero: nothing is pruned.
    const int x = tid >> 2, q4 = tid & 3;
    const uint32_t me = mx[x];
    uint32_t gt = 0u, ge = 0u;
    const LDS u32x4_t* m4 = reinterpret_cast<const LDS u32x4_t*>((const LDS uint32_t*)mx) + q4 * (kMaxSlabs / 16);
#pragma unroll
    for (int j = 0; j < kMaxSlabs / 16; ++j) {
      const u32x4_t y = m4[j];
      gt += (y.x > me) + (y.y > me) + (y.z > me) + (y.w > me);
      ge += (y.x >= me) + (y.y >= me) + (y.z >= me) + (y.w >= me);
    }
    gt += dpp<kDppXor1>(gt);
    gt += dpp<kDppXor2>(gt);
    ge += dpp<kDppXor1>(ge);
    ge += dpp<kDppXor2>(ge);
    if (q4 == 0 && (int)gt < K && (int)ge >= K) thr = me;
  }
  __syncthreads();
  const uint32_t T = thr;
  {
    // keys whose value word is >= T (non-zero) gathered into sv, one LDS
    // atomic a wave
    uint64_t bal[kMPer];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < kMPer; ++i) {
      bal[i] = __ballot((h[i] | l[i]) != 0u && h[i] >= T);
      tot += __popcll(bal[i]);
    }
    int base = 0;
    if (lane == 0 && tot) base = lds_add((LDS int*)&nsv, tot);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int i = 0; i < kMPer; ++i) {
      const int pos = base + (int)mbcnt64(bal[i]);
      if (((bal[i] >> lane) & 1ull) && pos < kSurvCap) sv[pos] = ((uint64_t)h[i] << 32) | l[i];
      base += __popcll(bal[i]);
    }
  }
  __syncthreads();
  const int ns = nsv;
  if (ns <= kSurvCap) {
    // rank by counting: a key's place is the number of larger survivors
    if (tid < ns) {
      const uint64_t me = sv[tid];
      uint32_t r = 0u;
      int j = 0;
      for (; j + 4 <= ns; j += 4) {
        uint64_t k4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) k4[e] = sv[j + e];
#pragma unroll
        for (int e = 0; e < 4; ++e) r += k4[e] > me ? 1u : 0u;
      }
      for (; j < ns; ++j) r += sv[j] > me ? 1u : 0u;
      if ((int)r < K) {
        cand_ids[(size_t)row * K + r] = (int32_t)(0xFFFFFFFFu - (uint32_t)me);
        cand_logit[(size_t)row * K + r] = key_to_f32((uint32_t)(me >> 32));
      }
    }
    // fewer than K keys in the row: the places past them are empty
    if (tid >= ns && tid < K) {
      cand_ids[(size_t)row * K + tid] = -1;
      cand_logit[(size_t)row * K + tid] = -__builtin_huge_valf();
    }
    return;
  }
  merge_tree16(h, l);
  part[w][lane] = ((uint64_t)h[0] << 32) | l[0];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < kMW; ++i) {
      const uint64_t x = part[i][lane];
      h[i] = (uint32_t)(x >> 32);
      l[i] = (uint32_t)x;
    }
    merge_tree16(h, l);
    if (v) {
      const bool ok = (h[0] | l[0]) != 0u;
      cand_ids[(size_t)row * K + lane] = ok ? (int32_t)(0xFFFFFFFFu - l[0]) : -1;
      cand_logit[(size_t)row * K + lane] = ok ? key_to_f32(h[0]) : -__builtin_huge_valf();
    }
  }
}

// Measurement utility (not a step of the method): reads n 16-byte vectors
// once, grid-stride, eight loads in flight a thread, and folds them into one
// word that is stored only if it matches an impossible pattern.
__global__ __launch_bounds__(512) void stream_read_kernel(const u32x4_t* __restrict__ p, size_t n, uint32_t* sink) {
  const size_t T = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 7 * T < n; i += 8 * T) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * T];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += T) {
    const u32x4_t v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;
}

// Measurement utility (not a step of the method): one workgroup of 1024
// threads reads n 16-byte vectors once, eight loads in flight a thread: the
// rate at which one CU pulls data from the memory system, the bound of a
// kernel that runs a request's whole round in one workgroup.
__global__ __launch_bounds__(1024) void cu_read_kernel(const u32x4_t* __restrict__ p, size_t n, uint32_t* sink) {
  constexpr size_t T = 1024;
  size_t i = threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 7 * T < n; i += 8 * T) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * T];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += T) {
    const u32x4_t v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;
}

}  // namespace

hipError_t launch_cu_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(cu_read_kernel, dim3(1), dim3(1024), 0, s, static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(256), dim3(512), 0, s, static_cast<const u32x4_t*>(buf), bytes / 16,
                     sink);
  return hipGetLastError();
}

LmheadPlan lmhead_plan(int rows, int V, int D, int K) {
  LmheadPlan p{};
  p.ok = false;
  if (rows < 1 || V < 1 || K < 1 || K > kWave || K > V || D < 256 || D % 256 != 0) return p;
  p.ntiles = (V + 15) / 16;
  p.S = min(kMaxSlabs, p.ntiles);
  const int tiles_per_slab = (p.ntiles + p.S - 1) / p.S;
  if (tiles_per_slab > kSlabTiles) return p;
  p.slab_cols = tiles_per_slab * 16;
  p.ring = D % 512 == 0 ? 16 : 8;
  const size_t fixed = (size_t)16 * (p.slab_cols + 4) * 4 + (size_t)kLW * kWave * 8;
  const int step = 32 * p.ring;
  // the largest chunk of D (a multiple of 32 * ring) whose staged rows fit
  int kc = D;
  while (kc > step && fixed + (size_t)16 * (kc + 8) * 2 > kLdsMax) kc -= step;
  if (fixed + (size_t)16 * (kc + 8) * 2 > kLdsMax) return p;
  p.kc = kc;
  p.smem = fixed + (size_t)16 * (kc + 8) * 2;
  p.list_bytes = (size_t)rows * p.S * K * sizeof(uint64_t);
  p.ok = true;
  return p;
}

hipError_t launch_lmhead_topk(const LmheadPlan& p, const uint16_t* X, const uint16_t* Wlm, int rows, int V, int D,
                              int K, uint64_t* lists, int32_t* cand_ids, float* cand_logit, hipStream_t s) {
  LmArgs a{};
  a.X = X;
  a.W = Wlm;
  a.rows = rows;
  a.V = V;
  a.D = D;
  a.K = K;
  a.S = p.S;
  a.ntiles = p.ntiles;
  a.kc = p.kc;
  a.slab_cols = p.slab_cols;
  a.lists = lists;
  const dim3 grid((unsigned)p.S, (unsigned)((rows + 15) / 16));
  const void* fn = p.ring == 16 ? (const void*)lmhead_topk_kernel<16> : (const void*)lmhead_topk_kernel<8>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.smem);
  if (e != hipSuccess) return e;
  if (p.ring == 16)
    hipLaunchKernelGGL((lmhead_topk_kernel<16>), grid, dim3(kLT), p.smem, s, a);
  else
    hipLaunchKernelGGL((lmhead_topk_kernel<8>), grid, dim3(kLT), p.smem, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lmhead_merge_kernel, dim3(rows), dim3(kMT), 0, s, lists, p.S, K, cand_ids, cand_logit);
  return hipGetLastError();
}

}  // namespace dartree
