// Steps a2..a5 in one 1024-thread workgroup per request: depth-by-depth
// batched correction scoring, s_beta with per-depth top-W, the deferred
// global top-B, breadth-first emission and the tree-attention mask.
//
// DARTree (marsggbo blog, section 3.1): at depth d every surviving parent of
// depth d-1 goes through the correction head in one batched call and scores
// its K candidates; s_beta(u_1..u_d) = sum_i log q_i(u_i) + beta * d with
// beta <= 0; each depth keeps its top W, forming a supertree; after
// construction the B best nodes are chosen in one pass (Lemma 1: for beta <=
// 0 this set is prefix-closed and equals best-first heap pops). Section 3.2:
// the tree is verified under a tree-attention mask. The head is the declared
// low-rank stand-in:
//   z[p][c] = Lbase_d[c] + <s_p, U[c]>, log q = log-softmax over the K
//             candidates (clamped to <= 0, so a child never outscores its
//             parent in fp32 and the selection stays prefix-closed);
//   s_child = tanh(A s_p + E[u] + h_d)           (needed when d < L).
// One comparator orders nodes: s_beta descending, depth ascending, token
// ascending, parent slot ascending.
//
// Contractions. bf16 weights run on v_mfma_f32_16x16x32_bf16 with each fp32
// state split exactly into three bf16 parts (hi + mid + lo == s), so every
// product is exact and only fp32 accumulation rounds; fp32 weights use FMAs.
// Mode 2 (r = 256, K <= 64, W <= 16, the block-decoding shapes) keeps A in
// registers (wave w owns rows 16w..16w+15), keeps the parents' split states in
// LDS, and prefetches the next depth's U fragments (registers), E rows and h
// row (LDS) while the current depth runs, so the dependent chain never waits
// on global memory. Mode 1 is the same arithmetic with loads issued per tile:
// weight fragments are read with 4-lane groups on one 64-byte segment and
// permuted to the operand lanes, and the parents' states are kept as split
// planes when they fit in LDS (else split per fragment from fp32 rows).
//
// Emission order (depth, parent's emitted index, token) equals the order of
// the nodes' token paths, so each level records the lexicographic rank of its
// nodes' paths and the emitted index of a selected node is its level's base
// plus the number of selected nodes of its level with a smaller path rank.
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / kWave;
constexpr int kSelCap = 1024;
constexpr size_t kMaxSmem = 160 * 1024;
constexpr int kGB = 8;   // mode 1: weight fragments in flight per tile batch

__device__ __forceinline__ float ldw(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldw(const float* p, size_t i) { return p[i]; }

// LDS row strides are padded so that the MFMA operand and result patterns
// (16 rows, same columns) fall into different banks: split states r + 8
// halves (16-byte reads of 8 consecutive rows cover all 32 banks), fp32
// states and A*S rows r + 1 floats, partial logits K + 4 floats.
// All pointers are LDS-qualified (address space 3) and held by value, so
// every access compiles to a ds_* instruction.
struct Lay {
  LDS int* cid;       // mode 2: [L][K]; else [K] (current depth)
  LDS float* clog;
  LDS float* Sf;      // mode 0, mode 1 without planes: [W][r+1] fp32 parent states
  LDS uint16_t* Sh;   // mode 2: [16][r+8], mode 1 with planes: [ceil16(W)][r+8] split parent states
  LDS uint16_t* Sm;
  LDS uint16_t* Sl;
  LDS float* Zp;      // [KQ][W][K+4] partial corrected logits; slice 0 then holds cum
  LDS float* AS;      // [W][r+1]
  LDS float* cumP;    // [W]
  LDS int* lv_tok;    // [L][W]
  LDS int* lv_ps;
  LDS int* lv_lex;
  LDS int* lv_k;
  LDS float* lv_cum;
  LDS float* lv_sb;
  LDS int* lv_cnt;    // [32]
  LDS uint16_t* EC;   // mode 2: [2][K][r]
  LDS float* hb;      // mode 2: [2][r]
  LDS uint64_t* skey; // [kSelCap]
  LDS int* spay;
  LDS uint64_t* okey; // [max(W, B)]
  LDS int* opay;
  LDS int* misc;      // [16]
  LDS int* eidx;      // [L][W]
  LDS int* eord;      // [B]
  LDS int* nd;        // [32]
  LDS int* base;      // [33]
  LDS int* epar;      // [B]
  LDS uint64_t* mb;   // [2][64]
  LDS int* ab;        // [2][64]
};

struct LayOff {
  size_t cid, clog, sf, sh, sm, sl, zp, as, cp, tok, ps, lex, k, cum, sb, cnt, ec, hb, sk, sp, ok, op, misc, eidx,
      eord, nd, base, epar, mb, ab, total;
};

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }

// pl: mode 1 keeps the parents' states as split planes of ceil16(W) rows
// (written once per state, read by every tile) instead of fp32 rows split on
// the fly per fragment.
__host__ __device__ inline LayOff lay_off(int L, int K, int W, int B, int r, int mode, int KQ, bool pl = false) {
  LayOff o{};
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t x = off;
    off = al16(off + b);
    return x;
  };
  const size_t LW = (size_t)L * W;
  const size_t ncand = mode == 2 ? (size_t)L * K : (size_t)K;
  const size_t outn = (size_t)(W > B ? W : B);
  o.cid = take(4 * ncand);
  o.clog = take(4 * ncand);
  const bool planes = mode == 2 || (mode == 1 && pl);
  const size_t prows = mode == 2 ? 16 : (size_t)(W + 15) / 16 * 16;
  o.sf = planes ? 0 : take(4ul * W * (r + 1));
  o.sh = planes ? take(2ul * prows * (r + 8)) : 0;
  o.sm = planes ? take(2ul * prows * (r + 8)) : 0;
  o.sl = planes ? take(2ul * prows * (r + 8)) : 0;
  o.zp = take(4ul * KQ * W * (K + 4));
  o.as = take(4ul * W * (r + 1));
  o.cp = take(4ul * W);
  o.tok = take(4 * LW);
  o.ps = take(4 * LW);
  o.lex = take(4 * LW);
  o.k = take(4 * LW);
  o.cum = take(4 * LW);
  o.sb = take(4 * LW);
  o.cnt = take(4 * 32);
  o.ec = mode == 2 ? take(2ul * 2 * K * r) : 0;
  o.hb = mode == 2 ? take(4ul * 2 * r) : 0;
  o.sk = take(8ul * kSelCap);
  o.sp = take(4ul * kSelCap);
  o.ok = take(8 * outn);
  o.op = take(4 * outn);
  o.misc = take(4 * 16);
  o.eidx = take(4 * LW);
  o.eord = take(4ul * B);
  o.nd = take(4 * 32);
  o.base = take(4 * 33);
  o.epar = take(4ul * B);
  o.mb = take(8 * 128);
  o.ab = take(4 * 128);
  o.total = off;
  return o;
}

__device__ __forceinline__ Lay make_lay(const LayOff& o) {
  extern __shared__ __align__(16) char smem[];
  LDS char* b = (LDS char*)smem;
  Lay s;
  s.cid = (LDS int*)(b + o.cid);
  s.clog = (LDS float*)(b + o.clog);
  s.Sf = (LDS float*)(b + o.sf);
  s.Sh = (LDS uint16_t*)(b + o.sh);
  s.Sm = (LDS uint16_t*)(b + o.sm);
  s.Sl = (LDS uint16_t*)(b + o.sl);
  s.Zp = (LDS float*)(b + o.zp);
  s.AS = (LDS float*)(b + o.as);
  s.cumP = (LDS float*)(b + o.cp);
  s.lv_tok = (LDS int*)(b + o.tok);
  s.lv_ps = (LDS int*)(b + o.ps);
  s.lv_lex = (LDS int*)(b + o.lex);
  s.lv_k = (LDS int*)(b + o.k);
  s.lv_cum = (LDS float*)(b + o.cum);
  s.lv_sb = (LDS float*)(b + o.sb);
  s.lv_cnt = (LDS int*)(b + o.cnt);
  s.EC = (LDS uint16_t*)(b + o.ec);
  s.hb = (LDS float*)(b + o.hb);
  s.skey = (LDS uint64_t*)(b + o.sk);
  s.spay = (LDS int*)(b + o.sp);
  s.okey = (LDS uint64_t*)(b + o.ok);
  s.opay = (LDS int*)(b + o.op);
  s.misc = (LDS int*)(b + o.misc);
  s.eidx = (LDS int*)(b + o.eidx);
  s.eord = (LDS int*)(b + o.eord);
  s.nd = (LDS int*)(b + o.nd);
  s.base = (LDS int*)(b + o.base);
  s.epar = (LDS int*)(b + o.epar);
  s.mb = (LDS uint64_t*)(b + o.mb);
  s.ab = (LDS int*)(b + o.ab);
  return s;
}

__device__ __forceinline__ void split_store(const Lay& s, int r, int row, int j, float v) {
  uint32_t h, m, l;
  split3(v, h, m, l);
  const int o = row * (r + 8) + j;
  s.Sh[o] = (uint16_t)h;
  s.Sm[o] = (uint16_t)m;
  s.Sl[o] = (uint16_t)l;
}

// three bf16 fragments of 8 consecutive fp32 values (split on the fly)
__device__ __forceinline__ void split_frag(const LDS float* src, bool valid, u16x8_t& fh, u16x8_t& fm, u16x8_t& fl) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t h, m, l;
    split3(valid ? src[i] : 0.f, h, m, l);
    fh[i] = (unsigned short)h;
    fm[i] = (unsigned short)m;
    fl[i] = (unsigned short)l;
  }
}

// ---- mode 1: MFMA with loads issued per tile ---------------------------------
// The three bf16 fragments of parent row p at columns j0..j0+7: read from the
// split planes (PL) or split from the fp32 row on the fly.
template <bool PL>
__device__ __forceinline__ void state_frag(const Lay& s, int r, int p, bool pv, int j0, u16x8_t& fh, u16x8_t& fm,
                                           u16x8_t& fl) {
  if (PL) {
    const int o = p * (r + 8) + j0;
    fh = *reinterpret_cast<const LDS u16x8_t*>(s.Sh + o);
    fm = *reinterpret_cast<const LDS u16x8_t*>(s.Sm + o);
    fl = *reinterpret_cast<const LDS u16x8_t*>(s.Sl + o);
  } else {
    split_frag(s.Sf + (size_t)(pv ? p : 0) * (r + 1) + j0, pv, fh, fm, fl);
  }
}

// Weight fragments of one tile are loaded GB k-steps at a time (all loads of
// a batch in flight together), then consumed in order.
// Z tiles of candidate blocks n0..n1-1 (16 candidates each); AS tiles of
// A-row blocks m0..m1-1. Tile t goes to wave (t + wofs) mod 16.
template <bool PL, int GB>
__device__ __forceinline__ void z_mfma_general(const Lay& s, const uint16_t* __restrict__ U, int Wp, int K, int r,
                                               int n0, int n1, int wofs) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int MT = (Wp + 15) / 16, NT = n1 - n0, KS = r / 32;
  const int sub = (lane >> 4) * 8;
  for (int t = (w + kWaves - wofs) % kWaves; t < MT * NT; t += kWaves) {
    const int mt = t / NT, nt = n0 + t % NT;
    const int p = mt * 16 + (lane & 15);
    const int k = nt * 16 + (lane & 15);
    const bool pv = p < Wp, kv = k < K;
    // coalesced rows; a candidate column >= K re-reads a valid row and feeds only discarded outputs
    const uint16_t* urow = U + (size_t)s.cid[min(nt * 16 + coal_row(lane), K - 1)] * r + coal_col(lane);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KS; k0 += GB) {
      // every load of the batch is issued (past the end it re-reads the last
      // k-step, unused), so the compiler waits for each fragment alone
      u16x8_t b[GB];
#pragma unroll
      for (int g = 0; g < GB; ++g) b[g] = *reinterpret_cast<const u16x8_t*>(urow + min(k0 + g, KS - 1) * 32);
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        if (k0 + g < KS) {
          b[g] = to_mfma_lanes(b[g], lane);
          u16x8_t fh, fm, fl;
          state_frag<PL>(s, r, p, pv, (k0 + g) * 32 + sub, fh, fm, fl);
          acc = mfma_bf16(fl, b[g], acc);
          acc = mfma_bf16(fm, b[g], acc);
          acc = mfma_bf16(fh, b[g], acc);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = mt * 16 + (lane >> 4) * 4 + i;
      if (pp < Wp && kv) s.Zp[pp * (K + 4) + k] = acc[i];
    }
  }
}

template <bool PL, int GB>
__device__ __forceinline__ void as_mfma_general(const Lay& s, const uint16_t* __restrict__ A, int Wp, int r, int m0,
                                                int m1, int wofs) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int MT = m1 - m0, NT = (Wp + 15) / 16, KS = r / 32;
  const int sub = (lane >> 4) * 8;
  for (int t = (w + kWaves - wofs) % kWaves; t < MT * NT; t += kWaves) {
    const int mt = m0 + t / NT, nt = t % NT;
    const int p = nt * 16 + (lane & 15);
    const bool pv = p < Wp;
    const uint16_t* arow = A + (size_t)(mt * 16 + coal_row(lane)) * r + coal_col(lane);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KS; k0 += GB) {
      u16x8_t av[GB];
#pragma unroll
      for (int g = 0; g < GB; ++g) av[g] = *reinterpret_cast<const u16x8_t*>(arow + min(k0 + g, KS - 1) * 32);
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        if (k0 + g < KS) {
          av[g] = to_mfma_lanes(av[g], lane);
          u16x8_t fh, fm, fl;
          state_frag<PL>(s, r, p, pv, (k0 + g) * 32 + sub, fh, fm, fl);
          acc = mfma_bf16(av[g], fl, acc);
          acc = mfma_bf16(av[g], fm, acc);
          acc = mfma_bf16(av[g], fh, acc);
        }
      }
    }
    if (pv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s.AS[p * (r + 1) + mt * 16 + (lane >> 4) * 4 + i] = acc[i];
    }
  }
}

// ---- mode 0: fp32 FMAs --------------------------------------------------------
template <typename WT>
__device__ __forceinline__ void z_valu(const Lay& s, const WT* __restrict__ U, int Wp, int K, int r) {
  for (int idx = threadIdx.x; idx < Wp * K; idx += kT) {
    const int p = idx / K, k = idx - p * K;
    const size_t ub = (size_t)s.cid[k] * r;
    const LDS float* srow = s.Sf + (size_t)p * (r + 1);
    float acc = 0.f;
    for (int j = 0; j < r; ++j) acc = fmaf(srow[j], ldw(U, ub + j), acc);
    s.Zp[p * (K + 4) + k] = acc;
  }
}
template <typename WT>
__device__ __forceinline__ void as_valu(const Lay& s, const WT* __restrict__ A, int Wp, int r) {
  for (int idx = threadIdx.x; idx < Wp * r; idx += kT) {
    const int p = idx / r, j = idx - p * r;
    const LDS float* srow = s.Sf + (size_t)p * (r + 1);
    float acc = 0.f;
    for (int m = 0; m < r; ++m) acc = fmaf(ldw(A, (size_t)j * r + m), srow[m], acc);
    s.AS[p * (r + 1) + j] = acc;
  }
}

// Lexicographic rank of each node's token path within its level: order of
// (parent's path rank, token) among the level's cnt nodes.
__device__ __forceinline__ void level_lex(const Lay& s, int d, int W, int cnt) {
  const int tid = threadIdx.x;
  if (tid < cnt) {
    const int row = (d - 1) * W;
    auto k2 = [&](int sl) {
      const int lp = d == 1 ? 0 : s.lv_lex[row - W + min(max(s.lv_ps[row + sl], 0), W - 1)];
      return (lp << 18) | (s.lv_tok[row + sl] & 0x3FFFF);
    };
    const int my = k2(tid);
    int rk = 0;
    for (int sl = 0; sl < cnt; ++sl) rk += k2(sl) < my;
    s.lv_lex[row + tid] = rk;
  }
}

template <typename WT, int MODE, int KSQ, int EPT, bool PL = false>
__global__ __launch_bounds__(kT) void tree_kernel(TreeArgs a, int KQ) {
  // split planes hold the parents' states (mode 2 always, mode 1 with PL)
  constexpr bool kPl = MODE == 2 || (MODE == 1 && PL);
  const Lay s = make_lay(lay_off(a.L, a.K, a.W, a.B, a.r, MODE, KQ, PL));
  // mode 1 may split a request over a.split workgroups (parts): part p
  // computes its share of the contraction tiles and publishes it; every part
  // then runs the same selection and state update; part 0 writes the outputs
  const int nsplit = MODE == 1 ? a.split : 1;
  const int q = blockIdx.x / nsplit, part = blockIdx.x % nsplit;
  const bool lead = part == 0;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int L = a.L, K = a.K, W = a.W, r = a.r, B = a.B;
  // this request's width and budget (per-request values clamped to [1, W], [1, B])
  const int Wq = a.w_req ? min(max(a.w_req[q], 1), W) : W;
  const int Bq = a.b_req ? min(max(a.b_req[q], 1), B) : B;
  const size_t lw = (size_t)q * L * W;
  const WT* A = static_cast<const WT*>(a.A);
  // no A: the Markov head, whose states have no recurrence (A s_parent = 0)
  const bool markov = A == nullptr;
  const WT* E = static_cast<const WT*>(a.E);
  const WT* U = static_cast<const WT*>(a.U);
  const float* hq = a.h + (size_t)q * L * r;
  const int32_t* cid_g = a.cand_ids + (size_t)q * L * K;
  const float* clog_g = a.cand_logit + (size_t)q * L * K;
  SelSmem sel{s.skey, s.spay, s.okey, s.opay, s.misc, kSelCap};
  const bool expand = a.d0 <= a.d1;

  if (tid < 16) s.misc[tid] = 0;
  for (int d = tid; d < 32; d += kT) s.lv_cnt[d] = d < L ? min(max(a.st_count[(size_t)q * L + d], 0), W) : 0;
  // levels this launch does not expand come from global memory
  for (int i = tid; i < L * W; i += kT) {
    const int d = i / W + 1;
    const bool here = expand && d >= a.d0 && d <= a.d1;
    if (!here && (a.do_select || (expand && d == a.d0 - 1))) {
      s.lv_tok[i] = a.st_tok[lw + i];
      s.lv_ps[i] = a.st_parent[lw + i];
      s.lv_sb[i] = a.st_sbeta[lw + i];
      s.lv_cum[i] = a.st_cum[lw + i];
    }
  }
  if (MODE == 2 && expand) {
    for (int i = tid; i < L * K; i += kT) {
      const int c = cid_g[i];
      s.cid[i] = (c < 0 || c >= a.V) ? 0 : c;
      s.clog[i] = clog_g[i];
    }
  }
  int Wp = 1;
  if (MODE == 1 && PL && expand) {
    // padding rows of the planes feed only discarded outputs; clear them anyway
    const int n = (W + 15) / 16 * 16 * (r + 8);
    for (int i = tid; i < n; i += kT) s.Sh[i] = s.Sm[i] = s.Sl[i] = 0;
    __syncthreads();
  }
  if (expand) {
    if (a.d0 == 1) {
      for (int j = tid; j < r; j += kT) {
        if (kPl) split_store(s, r, 0, j, hq[j]);
        else s.Sf[j] = hq[j];
      }
      if (tid == 0) s.cumP[0] = 0.f;
    } else {
      Wp = min(max(a.st_count[(size_t)q * L + a.d0 - 2], 1), W);
      const float* st = a.st_state + (size_t)q * W * r;
      for (int i = tid; i < Wp * r; i += kT) {
        if (kPl) split_store(s, r, i / r, i % r, st[i]);
        else s.Sf[(i / r) * (r + 1) + i % r] = st[i];
      }
      for (int i = tid; i < Wp; i += kT) s.cumP[i] = a.st_cum[lw + (size_t)(a.d0 - 2) * W + i];
    }
  }

  // ---- mode 2 register state: A rows of tile w, U fragments of this depth ----
  constexpr int NEV = 2;                 // E prefetch vectors per thread (K*r/8 <= 2048)
  u16x8_t areg[MODE == 2 ? 8 : 1];
  u16x8_t ureg[KSQ], unxt[KSQ];
  const int NT = K / 16;
  const int sub = (lane >> 4) * 8;
  const bool zw = MODE == 2 && w < NT * KQ;   // this wave computes a Z tile
  const int z_nt = MODE == 2 ? w % (NT > 0 ? NT : 1) : 0;
  const int z_kq = MODE == 2 ? w / (NT > 0 ? NT : 1) : 0;
  auto load_u = [&](u16x8_t (&dst)[KSQ], int d) {
    if (zw) {
      const int row = s.cid[(d - 1) * K + z_nt * 16 + (lane & 15)];
      const uint16_t* src = reinterpret_cast<const uint16_t*>(U) + (size_t)row * r + sub;
#pragma unroll
      for (int i = 0; i < KSQ; ++i) dst[i] = *reinterpret_cast<const u16x8_t*>(src + (z_kq * KSQ + i) * 32);
    }
  };
  // E rows of depth d's candidates and h_d go straight from global memory to
  // LDS (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at the
  // wave's base + 16 l), no registers involved.
  const int nvec_e = K * r / 8;
  auto load_e = [&](int d) {
    LDS uint16_t* ebuf = s.EC + (size_t)(d & 1) * K * r;
#pragma unroll
    for (int i = 0; i < NEV; ++i) {
      const int v0 = w * kWave + i * kT;   // first vector of this wave
      const int v = v0 + lane;
      if (v < nvec_e) {
        const int k = v / (r / 8), c = (v % (r / 8)) * 8;
        const int row = s.cid[(d - 1) * K + k];
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(E) + (size_t)row * r + c, ebuf + (size_t)v0 * 8,
                                         16, 0, 0);
      }
    }
    if (w == 0)
      __builtin_amdgcn_global_load_lds(hq + (size_t)d * r + lane * 4, s.hb + (size_t)(d & 1) * r, 16, 0, 0);
  };
  if (MODE == 2 && expand) {
    __syncthreads();   // candidates in LDS
    const uint16_t* arow = reinterpret_cast<const uint16_t*>(A) + (size_t)(w * 16 + (lane & 15)) * r + sub;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      areg[ks] = markov ? u16x8_t{0, 0, 0, 0, 0, 0, 0, 0} : *reinterpret_cast<const u16x8_t*>(arow + ks * 32);
    load_u(ureg, a.d0);
    if (a.d0 < L) load_e(a.d0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the LDS-direct loads have landed
  }
  // modes 0/1: candidates of the first depth (later depths are loaded one depth ahead)
  int c_nx = 0;
  float l_nx = 0.f;
  if (MODE != 2 && expand && tid < K) {
    c_nx = cid_g[(size_t)(a.d0 - 1) * K + tid];
    l_nx = clog_g[(size_t)(a.d0 - 1) * K + tid];
  }
  __syncthreads();

  for (int d = a.d0; d <= a.d1; ++d) {
    const bool need_state = d < L;
    const LDS int* cidd = MODE == 2 ? s.cid + (size_t)(d - 1) * K : s.cid;
    const LDS float* clogd = MODE == 2 ? s.clog + (size_t)(d - 1) * K : s.clog;
    if (MODE != 2) {
      // this depth's candidates came in during the previous depth (K <= kT)
      if (tid < K) {
        s.cid[tid] = (c_nx < 0 || c_nx >= a.V) ? 0 : c_nx;
        s.clog[tid] = l_nx;
        if (d < a.d1) {
          c_nx = cid_g[(size_t)d * K + tid];
          l_nx = clog_g[(size_t)d * K + tid];
        }
      }
      __syncthreads();
    }
    // ---- contractions: Z = S U_C^T (partials) and AS = A S^T --------------
    if (MODE == 2) {
      if (zw) {
        const int p = lane & 15;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KSQ; ++i) {
          const int j0 = (z_kq * KSQ + i) * 32 + sub;
          const u16x8_t fh = *reinterpret_cast<const LDS u16x8_t*>(s.Sh + p * (r + 8) + j0);
          const u16x8_t fm = *reinterpret_cast<const LDS u16x8_t*>(s.Sm + p * (r + 8) + j0);
          const u16x8_t fl = *reinterpret_cast<const LDS u16x8_t*>(s.Sl + p * (r + 8) + j0);
          acc = mfma_bf16(fl, ureg[i], acc);
          acc = mfma_bf16(fm, ureg[i], acc);
          acc = mfma_bf16(fh, ureg[i], acc);
        }
        const int k = z_nt * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pp = (lane >> 4) * 4 + i;
          if (pp < Wp) s.Zp[((size_t)z_kq * W + pp) * (K + 4) + k] = acc[i];
        }
      }
      if (need_state && !markov) {
        const int p = lane & 15;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int m0 = ks * 32 + sub;
          const u16x8_t fh = *reinterpret_cast<const LDS u16x8_t*>(s.Sh + p * (r + 8) + m0);
          const u16x8_t fm = *reinterpret_cast<const LDS u16x8_t*>(s.Sm + p * (r + 8) + m0);
          const u16x8_t fl = *reinterpret_cast<const LDS u16x8_t*>(s.Sl + p * (r + 8) + m0);
          acc = mfma_bf16(areg[ks], fl, acc);
          acc = mfma_bf16(areg[ks], fm, acc);
          acc = mfma_bf16(areg[ks], fh, acc);
        }
        if (p < Wp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s.AS[p * (r + 1) + w * 16 + (lane >> 4) * 4 + i] = acc[i];
        }
      }
      if (d < a.d1) {
        load_u(unxt, d + 1);
        if (d + 1 < L) load_e(d + 1);
      }
    } else if (MODE == 1) {
      const uint16_t* U16 = reinterpret_cast<const uint16_t*>(U);
      const uint16_t* A16 = reinterpret_cast<const uint16_t*>(A);
      const bool with_as = need_state && !markov;
      const int NZ = (K + 15) / 16, NA = r / 16;
      auto z_of = [&](int pt, int& n0, int& n1) {
        n0 = NZ * pt / nsplit;
        n1 = NZ * (pt + 1) / nsplit;
      };
      auto a_of = [&](int pt, int& m0, int& m1) {
        m0 = NA * pt / nsplit;
        m1 = NA * (pt + 1) / nsplit;
      };
      // a part's tiles: Z on waves 0.., then AS on the following waves
      auto contract = [&](int pt) {
        int n0, n1, m0, m1;
        z_of(pt, n0, n1);
        a_of(pt, m0, m1);
        z_mfma_general<PL, kGB>(s, U16, Wp, K, r, n0, n1, 0);
        if (with_as) as_mfma_general<PL, kGB>(s, A16, Wp, r, m0, m1, ((Wp + 15) / 16 * (n1 - n0)) % kWaves);
      };
      contract(part);
      if (nsplit > 1) {
        // Publish this part's Z and AS columns, then raise its flag. An
        // exchange row holds the Z columns in 16-column blocks (NZ * 16,
        // columns >= K unused) and then the r AS columns; rows of a (request,
        // depth) are consecutive. Slices move as 16-byte buffer accesses with
        // the sc1 policy (coherent across the XCDs' L2 caches, as the agent-
        // scope atomics are); the flag goes up once every wave's stores have
        // completed.
        __syncthreads();
        const int XS = NZ * 16 + r;
        float* xd = a.xch + ((size_t)q * L + d - 1) * W * XS;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(xd, 0, W * XS * 4, 0x00020000);
        int n0, n1, m0, m1;
        z_of(part, n0, n1);
        a_of(part, m0, m1);
        {
          const int nz4 = (n1 - n0) * 4, na4 = with_as ? (m1 - m0) * 4 : 0, nv = nz4 + na4;
          for (int i = tid; i < Wp * nv; i += kT) {
            const int p = i / nv, c = i - p * nv;
            const int col = c < nz4 ? n0 * 16 + 4 * c : NZ * 16 + m0 * 16 + 4 * (c - nz4);
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = c < nz4 ? (col + e < K ? s.Zp[p * (K + 4) + col + e] : 0.f) : s.AS[p * (r + 1) + col - NZ * 16 + e];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), xr, (p * XS + col) * 4, 0, 16);
          }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        uint32_t* fl = a.xflag + (size_t)q * nsplit * L;
        if (tid == 0) __hip_atomic_store(fl + (size_t)part * L + d - 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the other parts' flags, each waited for at most a.split_wait ticks of
        // the 100 MHz wall clock; a part that has not published (not resident,
        // or preempted) is computed here, and not waited for again in this launch
        if (tid < nsplit && tid != part) {
          int ok = 0;
          if (!((s.misc[11] >> tid) & 1)) {
            const uint32_t* f = fl + (size_t)tid * L + d - 1;
            const uint64_t t0 = wall_clock64();
            while (true) {
              if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                ok = 1;
                break;
              }
              if (wall_clock64() - t0 >= (uint64_t)a.split_wait) break;
              __builtin_amdgcn_s_sleep(2);
            }
            if (!ok) lds_or(&s.misc[11], 1 << tid);
          }
          s.misc[12 + tid] = ok;
        }
        asm volatile("" ::: "memory");
        __syncthreads();
        // the published slices of the other parts, in batches of kG vectors a
        // thread (one batch at most shapes: W (K + r) <= 16384 columns in all,
        // three quarters of them from the other parts, plus the rounding of
        // the parts' block ranges); a batch's loads are all issued before its
        // LDS writes, and an index past the end re-reads the last vector
        int beg[5], c0[4], nz4[4], nv[4];
        int total = 0;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          beg[pt] = total;
          c0[pt] = nz4[pt] = nv[pt] = 0;
          if (pt < nsplit && pt != part && s.misc[12 + pt]) {
            z_of(pt, n0, n1);
            a_of(pt, m0, m1);
            nz4[pt] = (n1 - n0) * 4;
            nv[pt] = nz4[pt] + (with_as ? (m1 - m0) * 4 : 0);
            c0[pt] = (n0 << 16) | (m0 * 16);   // first Z block, first AS column
            total += Wp * nv[pt];
          }
        }
        beg[4] = total;
        auto item = [&](int i, int& p, int& col) {
          const int pt = i < beg[1] ? 0 : i < beg[2] ? 1 : i < beg[3] ? 2 : 3;
          const int j = i - beg[pt];
          p = j / nv[pt];
          const int c = j - p * nv[pt];
          col = c < nz4[pt] ? (c0[pt] >> 16) * 16 + 4 * c : NZ * 16 + (c0[pt] & 0xFFFF) + 4 * (c - nz4[pt]);
        };
        constexpr int kG = 3;
        for (int i0 = 0; i0 < total; i0 += kG * kT) {
          f32x4_t gv[kG];
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            int p, col;
            item(min(i0 + tid + u * kT, total - 1), p, col);
            gv[u] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, (p * XS + col) * 4, 0, 16));
          }
#pragma unroll
          for (int u = 0; u < kG; ++u) {
            if (i0 + tid + u * kT < total) {
              int p, col;
              item(i0 + tid + u * kT, p, col);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (col < NZ * 16) {
                  if (col + e < K) s.Zp[p * (K + 4) + col + e] = gv[u][e];
                } else {
                  s.AS[p * (r + 1) + col - NZ * 16 + e] = gv[u][e];
                }
              }
            }
          }
        }
        for (int pt = 0; pt < nsplit; ++pt)
          if (pt != part && !s.misc[12 + pt]) contract(pt);
      }
    } else {
      z_valu<WT>(s, U, Wp, K, r);
      if (need_state && !markov) as_valu<WT>(s, A, Wp, r);
    }
    __syncthreads();

    // ---- log-softmax over the K candidates, cum, keys and the bound ---------
    const float bd = a.beta * (float)d;
    const int KJ = (K + kWave - 1) / kWave;
    uint64_t keys[EPT];
    int pays[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      keys[e] = 0ull;
      pays[e] = 0;
    }
    const int PJ = (Wp + kWaves - 1) / kWaves;
    for (int jp = 0; jp < PJ; ++jp) {
      const int p = w + jp * kWaves;
      if (p >= Wp) break;   // wave-uniform
      float z[EPT];
      float m = -__builtin_huge_valf();
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int k = lane + j * kWave;
        z[j] = -__builtin_huge_valf();
        if (j < KJ && k < K) {
          float v = 0.f;
          for (int qq = 0; qq < KQ; ++qq) v += s.Zp[((size_t)qq * W + p) * (K + 4) + k];
          z[j] = v + clogd[k];
          m = fmaxf(m, z[j]);
        }
      }
      m = wave_max_f32(m);
      // exp and log on the hardware exp2 / log2 with the change of base by
      // one multiply (relative error about 1e-7; the terms near the maximum
      // dominate the sum)
      float ssum = 0.f;
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if (j < KJ && lane + j * kWave < K) ssum += __builtin_amdgcn_exp2f((z[j] - m) * 1.4426950408889634f);
      ssum = wave_sum_f32(ssum);
      const float lse = m + __builtin_amdgcn_logf(ssum) * 0.6931471805599453f;
      const float cp = s.cumP[p];
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int k = lane + j * kWave;
        const int e = jp * KJ + j;
        if (j < KJ && k < K && e < EPT) {
          const float cum = cp + fminf(z[j] - lse, 0.f);
          s.Zp[(size_t)p * (K + 4) + k] = cum;
          const float sb = cum + bd;
          keys[e] = ((uint64_t)f32_key(sb) << 32) |
                    (uint64_t)(0xFFFFFFFFu - ((((uint32_t)cidd[k]) << 9) | (uint32_t)p));
          pays[e] = p * K + k;
        }
      }
    }
    {
      uint32_t lmax = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) lmax = max(lmax, (uint32_t)(keys[e] >> 32));
      const int nwk = min(kWaves, Wp);
      const int m = (W + nwk - 1) / nwk;
      if (w < nwk) {
        const bool v = lmax != 0u;
        const int nv = __popcll(__ballot(v));
        if (nv >= m && m <= kWave) {
          const uint32_t t = wave_mth_largest(lmax, v, m, 32);
          if (lane == 0) lds_max((LDS unsigned*)&s.misc[2], ~t);
        } else if (lane == 0) {
          lds_or(&s.misc[4], 1);
        }
        // A second bound: a wave holds Wq keys at or above the Wq-th largest
        // of its lane maxima. Wave 0 holds the best parent's children (the
        // parents are in rank order), whose Wq-th is usually far above the
        // first bound (the least of the waves' best keys): tens of survivors
        // instead of hundreds to rank. Taken from wave 0 alone, through the
        // 64-lane sort network, so the other waves do not wait on it.
        if (w == 0 && nv >= Wq && Wq <= kWave) {
          const uint32_t t2 = wave_mth_largest_sorted(lmax, v, Wq);
          if (lane == 0) lds_max((LDS unsigned*)&s.misc[6], t2);
        }
      }
    }
    __syncthreads();
    const uint32_t thr = max(s.misc[4] ? 0u : ~(uint32_t)s.misc[2], (uint32_t)s.misc[6]);
    int ns = select_compact<EPT>(keys, pays, thr, sel);
    if (ns > kSelCap) ns = select_exact<EPT>(keys, pays, Wq, sel);
    const int nk = select_rank(ns, Wq, sel);

    // mode 1: thread tid owns entries 8j..8j+7 of survivor sl's new state (W r
    // <= 8192 makes one vector per thread enough); its E row and h row loads go
    // out now and land while the new level is written
    const int r8 = r / 8;
    const bool sv = MODE == 1 && need_state && tid < nk * r8;
    int sv_sl = 0, sv_j0 = 0, sv_ps = 0;
    u16x8_t ev8 = {0, 0, 0, 0, 0, 0, 0, 0};
    float hv8[8];
    if (MODE == 1 && sv) {
      sv_sl = tid / r8;
      sv_j0 = (tid - sv_sl * r8) * 8;
      const int i = s.opay[sv_sl];
      sv_ps = i / K;
      const int tok = cidd[i - sv_ps * K];
      ev8 = *reinterpret_cast<const u16x8_t*>(reinterpret_cast<const uint16_t*>(E) + (size_t)tok * r + sv_j0);
      const float* hd = hq + (size_t)d * r + sv_j0;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv8[e] = hd[e];
    }

    // ---- the new level --------------------------------------------------------
    const size_t orow = lw + (size_t)(d - 1) * W;
    for (int sl = tid; sl < W; sl += kT) {
      if (sl < nk) {
        const int i = s.opay[sl];
        const int p = i / K, k = i - p * K;
        const float cum = s.Zp[(size_t)p * (K + 4) + k];
        const float sb = cum + bd;
        const int row = (d - 1) * W + sl;
        s.lv_tok[row] = cidd[k];
        s.lv_ps[row] = p;
        s.lv_k[row] = k;
        s.lv_cum[row] = cum;
        s.lv_sb[row] = sb;
        if (lead) {
          a.st_tok[orow + sl] = cidd[k];
          a.st_parent[orow + sl] = d == 1 ? 0 : p;
          a.st_cum[orow + sl] = cum;
          a.st_sbeta[orow + sl] = sb;
        }
      } else if (lead) {
        a.st_tok[orow + sl] = -1;
        a.st_parent[orow + sl] = -1;
        a.st_cum[orow + sl] = -__builtin_huge_valf();
        a.st_sbeta[orow + sl] = -__builtin_huge_valf();
      }
    }
    if (tid == 0) {
      s.lv_cnt[d - 1] = nk;
      if (lead) a.st_count[(size_t)q * L + d - 1] = nk;
    }
    if (MODE == 2) __builtin_amdgcn_s_waitcnt(0x0F70);   // next depth's E rows and h row have landed
    __syncthreads();

    // ---- head states of the survivors, their cum, path ranks -----------------
    if (need_state) {
      const float* hd = hq + (size_t)d * r;
      float* st_out = a.st_state + (size_t)q * W * r;
      const int row0 = (d - 1) * W;
      if (MODE == 1 && sv) {
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v8[e] = tanh_fast(((markov ? 0.f : s.AS[(size_t)sv_ps * (r + 1) + sv_j0 + e]) + bf16_to_f32(ev8[e])) + hv8[e]);
        if (kPl) {
          u16x8_t fh, fm, fl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t h, m, l;
            split3(v8[e], h, m, l);
            fh[e] = (unsigned short)h;
            fm[e] = (unsigned short)m;
            fl[e] = (unsigned short)l;
          }
          const int o = sv_sl * (r + 8) + sv_j0;
          *reinterpret_cast<LDS u16x8_t*>(s.Sh + o) = fh;
          *reinterpret_cast<LDS u16x8_t*>(s.Sm + o) = fm;
          *reinterpret_cast<LDS u16x8_t*>(s.Sl + o) = fl;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) s.Sf[sv_sl * (r + 1) + sv_j0 + e] = v8[e];
        }
        if (d == a.d1 && lead) {
#pragma unroll
          for (int e = 0; e < 8; ++e) st_out[(size_t)sv_sl * r + sv_j0 + e] = v8[e];
        }
      }
      for (int i = tid; MODE != 1 && i < nk * r; i += kT) {
        const int sl = i / r, j = i - sl * r;
        const int ps = s.lv_ps[row0 + sl];
        float ev, hv;
        if (MODE == 2) {
          ev = bf16_to_f32(s.EC[(size_t)(d & 1) * K * r + (size_t)s.lv_k[row0 + sl] * r + j]);
          hv = s.hb[(size_t)(d & 1) * r + j];
        } else {
          ev = ldw(E, (size_t)s.lv_tok[row0 + sl] * r + j);
          hv = hd[j];
        }
        const float v = tanh_fast(((markov ? 0.f : s.AS[(size_t)ps * (r + 1) + j]) + ev) + hv);
        if (kPl) split_store(s, r, sl, j, v);
        else s.Sf[sl * (r + 1) + j] = v;
        if (d == a.d1) st_out[i] = v;
      }
      for (int sl = tid; sl < nk; sl += kT) s.cumP[sl] = s.lv_cum[row0 + sl];
    }
    if (a.do_select && a.d0 == 1) level_lex(s, d, W, nk);
    Wp = nk;
    if (MODE == 2) {
#pragma unroll
      for (int i = 0; i < KSQ; ++i) ureg[i] = unxt[i];
    }
    __syncthreads();
  }

  if (!a.do_select || !lead) return;

  // ---- deferred global top-B ---------------------------------------------------
  if (!(expand && a.d0 == 1)) {
    for (int d = 1; d <= L; ++d) {
      level_lex(s, d, W, s.lv_cnt[d - 1]);
      __syncthreads();
    }
  }
  for (int i = tid; i < L * W; i += kT) s.eidx[i] = -1;
  for (int d = tid; d < 32; d += kT) s.nd[d] = 0;
  uint64_t keys[2];
  int pays[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = tid + e * kT;
    keys[e] = 0ull;
    pays[e] = i;
    if (i < L * W) {
      const int d = i / W + 1, sl = i - (d - 1) * W;
      if (sl < s.lv_cnt[d - 1]) {
        const uint32_t tok = (uint32_t)s.lv_tok[i] & 0x3FFFFu;
        const uint32_t ps = d == 1 ? 0u : ((uint32_t)s.lv_ps[i] & 0x1FFu);
        keys[e] = ((uint64_t)f32_key(s.lv_sb[i]) << 32) |
                  (uint64_t)(0xFFFFFFFFu - (((uint32_t)d << 27) | (tok << 9) | ps));
      }
    }
  }
  const int n = block_select<2>(keys, pays, Bq, 32, sel);
  for (int rr = tid; rr < n; rr += kT) {
    const int i = s.opay[rr];
    s.eidx[i] = 0;
    lds_add(&s.nd[i / W], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int d = 0; d < L; ++d) {
      s.base[d] = acc;
      acc += s.nd[d];
    }
    s.base[L] = acc;
  }
  __syncthreads();
  // emitted index: level base + selected nodes of the level with a smaller path
  for (int rr = tid; rr < n; rr += kT) {
    const int i = s.opay[rr];
    const int d = i / W + 1;
    const int row = (d - 1) * W, cnt = s.lv_cnt[d - 1];
    const int my = s.lv_lex[i];
    int rk = 0;
    for (int sl = 0; sl < cnt; ++sl) rk += (s.eidx[row + sl] >= 0) && (s.lv_lex[row + sl] < my);
    s.eord[rr] = s.base[d - 1] + rk;
  }
  __syncthreads();
  for (int rr = tid; rr < n; rr += kT) s.eidx[s.opay[rr]] = s.eord[rr];
  __syncthreads();
  int32_t* o_tok = a.tok + (size_t)q * B;
  int32_t* o_dep = a.depth + (size_t)q * B;
  int32_t* o_par = a.parent + (size_t)q * B;
  float* o_sc = a.score + (size_t)q * B;
  int32_t* o_slot = a.slot + (size_t)q * B;
  for (int rr = tid; rr < n; rr += kT) {
    const int i = s.opay[rr];
    const int d = i / W + 1, sl = i - (d - 1) * W;
    const int e = s.eidx[i];
    const int pe = d == 1 ? -1 : s.eidx[(d - 2) * W + min(max(s.lv_ps[i], 0), W - 1)];
    o_tok[e] = s.lv_tok[i];
    o_dep[e] = d;
    o_par[e] = pe;
    o_sc[e] = s.lv_sb[i];
    o_slot[e] = sl;
    s.epar[e] = pe;
  }
  for (int i = n + tid; i < B; i += kT) {
    o_tok[i] = -1;
    o_dep[i] = 0;
    o_par[i] = -2;
    o_sc[i] = -__builtin_huge_valf();
    o_slot[i] = -1;
  }
  if (tid == 0) a.n_sel[q] = n;
  if (!a.do_mask) return;
  __syncthreads();

  // ---- ancestor mask ------------------------------------------------------------
  const int words = (B + 63) / 64;
  uint64_t* mq = a.mask + (size_t)q * B * words;
  if (words == 1) {
    // pointer doubling: after round k, mb covers a node and its 2^k - 1
    // nearest ancestors and ab points at its 2^k-th ancestor
    if (tid < 64) {
      s.mb[tid] = tid < n ? (1ull << tid) : 0ull;
      s.ab[tid] = tid < n ? s.epar[tid] : -1;
    }
    __syncthreads();
    int cur = 0;
    for (int span = 1; span < L; span *= 2) {
      if (tid < 64) {
        const int an = s.ab[cur * 64 + tid];
        uint64_t mm = s.mb[cur * 64 + tid];
        int nx = -1;
        if (an >= 0 && an < tid) {
          mm |= s.mb[cur * 64 + an];
          nx = s.ab[cur * 64 + an];
        }
        s.mb[(cur ^ 1) * 64 + tid] = mm;
        s.ab[(cur ^ 1) * 64 + tid] = nx;
      }
      __syncthreads();
      cur ^= 1;
    }
    if (tid < B) mq[tid] = s.mb[cur * 64 + tid];
  } else {
    for (int t = tid; t < B * words; t += kT) {
      const int i = t / words, wd = t - i * words;
      uint64_t bits = 0ull;
      if (i < n) {
        int j = i;
        for (int step = 0; step <= L && j >= 0; ++step) {
          if ((j >> 6) == wd) bits |= 1ull << (j & 63);
          const int pj = s.epar[j];
          if (pj >= j || pj < -1) break;
          j = pj;
        }
      }
      mq[t] = bits;
    }
  }
}

// Standalone mask over arbitrary parent arrays: one thread per (row, word);
// walks follow only pointers with -1 <= parent[j] < j and stop after B steps.
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

TreePlan tree_plan(const TreeArgs& a) {
  const TreePlan f = tree_fast_plan(a);
  if (f.ok) return f;
  TreePlan p{};
  const bool al = ((((uintptr_t)a.A) | ((uintptr_t)a.E) | ((uintptr_t)a.U)) & 15u) == 0;
  int mode = 0;
  if (a.bf16 && a.r % 32 == 0 && al) mode = 1;
  int KQ = 1;
  if (mode == 1 && a.r == 256 && (a.K == 16 || a.K == 32 || a.K == 64) && a.W <= 16) {
    const int NT = a.K / 16;
    KQ = min(16 / NT, 8);
    const size_t sm2 = lay_off(a.L, a.K, a.W, a.B, a.r, 2, KQ).total;
    if (sm2 <= kMaxSmem) mode = 2;
    else KQ = 1;
  }
  p.mode = mode;
  p.kq = KQ;
  p.planes = mode == 1 && lay_off(a.L, a.K, a.W, a.B, a.r, 1, KQ, true).total <= kMaxSmem;
  p.split = (mode == 1 && a.split > 1 && a.xch && a.xflag) ? a.split : 1;
  p.smem = lay_off(a.L, a.K, a.W, a.B, a.r, mode, KQ, p.planes).total;
  p.ok = p.smem <= kMaxSmem;
  return p;
}

hipError_t launch_tree(const TreePlan& p, const TreeArgs& a0, hipStream_t s) {
  if (p.mode == 3) return launch_tree_fast(p, a0, s);
  TreeArgs a = a0;
  a.split = p.mode == 1 ? p.split : 1;
  dim3 grid(a.n_req * a.split), block(kT);
  hipError_t e = hipSuccess;
#define DT_TREE(T, M, KS, ...)                                                                             \
  do {                                                                                                     \
    e = hipFuncSetAttribute((const void*)tree_kernel<T, M, KS, __VA_ARGS__>,                               \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.smem);                      \
    if (e != hipSuccess) return e;                                                                         \
    hipLaunchKernelGGL((tree_kernel<T, M, KS, __VA_ARGS__>), grid, block, p.smem, s, a, p.kq);             \
  } while (0)
  if (p.mode == 2) {
    const int ksq = 8 / p.kq;
    if (ksq == 1) DT_TREE(uint16_t, 2, 1, 1);
    else DT_TREE(uint16_t, 2, 2, 1);
  } else {
    // keys per thread: parents per wave times 64-lane groups of candidates
    const int ept = ((a.W + kWaves - 1) / kWaves) * ((a.K + kWave - 1) / kWave);
    if (p.mode == 1 && p.planes) {
      if (ept <= 4) DT_TREE(uint16_t, 1, 1, 4, true);
      else if (ept <= 8) DT_TREE(uint16_t, 1, 1, 8, true);
      else DT_TREE(uint16_t, 1, 1, 16, true);
    } else if (p.mode == 1) {
      if (ept <= 4) DT_TREE(uint16_t, 1, 1, 4);
      else if (ept <= 8) DT_TREE(uint16_t, 1, 1, 8);
      else DT_TREE(uint16_t, 1, 1, 16);
    } else if (a.bf16) {
      if (ept <= 4) DT_TREE(uint16_t, 0, 1, 4);
      else if (ept <= 8) DT_TREE(uint16_t, 0, 1, 8);
      else DT_TREE(uint16_t, 0, 1, 16);
    } else {
      if (ept <= 4) DT_TREE(float, 0, 1, 4);
      else if (ept <= 8) DT_TREE(float, 0, 1, 8);
      else DT_TREE(float, 0, 1, 16);
    }
  }
#undef DT_TREE
  return hipGetLastError();
}

hipError_t launch_mask(int n_req, int B, const int32_t* n_sel, const int32_t* parent, uint64_t* mask,
                       hipStream_t s) {
  const int words = (B + 63) / 64;
  const int gx = (B * words + 255) / 256;
  hipLaunchKernelGGL(mask_kernel, dim3(gx, n_req), dim3(256), sizeof(int) * B, s, B, n_sel, parent, mask);
  return hipGetLastError();
}

namespace {

// 1 when either bf16 half of x has magnitude >= 2^16 (exponent field >= 143:
// beyond fp16's largest finite value; infinities and NaNs included)
__device__ __forceinline__ bool beyond_f16(uint32_t x) {
  return (x & 0x7FFFu) >= 0x4780u || ((x >> 16) & 0x7FFFu) >= 0x4780u;
}

__global__ __launch_bounds__(256) void head_check_kernel(const uint16_t* __restrict__ A, size_t nA,
                                                         const uint16_t* __restrict__ U, size_t nU,
                                                         int32_t* __restrict__ flags) {
  const size_t T = (size_t)gridDim.x * blockDim.x, t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  int f = 0;
  // whole 16-byte vectors, then the elements of a ragged end
  const size_t vA = nA / 8, vU = nU / 8;
  for (size_t i = t0; i < vU; i += T) {
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(U)[i];
    if (beyond_f16(v.x) || beyond_f16(v.y) || beyond_f16(v.z) || beyond_f16(v.w)) f |= 2;
  }
  for (size_t i = vU * 8 + t0; i < nU; i += T)
    if (beyond_f16(U[i])) f |= 2;
  if (A) {
    for (size_t i = t0; i < vA; i += T) {
      const u32x4_t v = reinterpret_cast<const u32x4_t*>(A)[i];
      if (beyond_f16(v.x) || beyond_f16(v.y) || beyond_f16(v.z) || beyond_f16(v.w)) f |= 1;
    }
    for (size_t i = vA * 8 + t0; i < nA; i += T)
      if (beyond_f16(A[i])) f |= 1;
  }
  // one global atomic a wave, and only from a wave that found something
  const int wf = (__ballot(f & 1) ? 1 : 0) | (__ballot(f & 2) ? 2 : 0);
  if (wf && lane_id() == 0) __hip_atomic_fetch_or(flags, wf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_head_check(const uint16_t* A, const uint16_t* U, int V, int r, int32_t* flags, hipStream_t s) {
  hipError_t e = launch_fill_u32(flags, 1, 0u, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_check_kernel, dim3(1024), dim3(256), 0, s, A, A ? (size_t)r * r : 0, U, (size_t)V * r,
                     flags);
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
