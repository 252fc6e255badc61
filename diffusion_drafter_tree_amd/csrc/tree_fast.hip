// Steps a2..a5 for the block-decoding shapes: bf16 weights, state width
// r = 256, K in {16, 32, 64} candidates per position, W <= 16 per depth.
// One 1024-thread workgroup per request, arranged for latency: five LDS-only
// barriers per depth and no wait on global memory inside the depth loop.
//
// DARTree (marsggbo blog, section 3.1): at depth d the surviving parents of
// depth d-1 are scored in one batched head call against their K candidates;
// s_beta = sum of log q + beta * d; each depth keeps its W best (the
// supertree); the B best supertree nodes are then taken in one pass, which is
// prefix-closed for beta <= 0 (Lemma 1). Section 3.2: the draft tree is
// verified under an ancestor mask. Node order everywhere: s_beta descending,
// then depth, token and parent slot ascending.
//
// Numerics: parent states as two fp16 planes (hi + lo, within 2^-20 of the
// fp32 state; the root state h_0 scaled by a power of two into fp16 range
// first), weights as fp16: exact for bf16 values of magnitude in
// [2^-17, 2^16) or zero, smaller ones truncated by at most 2^-25, and values
// of magnitude 2^16 or more beyond fp16's range -- a head with such A or U
// entries must go to the general kernel (DARTREE_HEAD_EXACT, found by
// dartree_head_check). Products on v_mfma_f32_16x16x32_f16 with fp32
// accumulation; fp32 log-softmax on the hardware exp2 / log2.
//
// Prologue: the scan's sorted slice lists merged per row (one wave per row),
// A fragments from the fp16 copy the scan launch staged, the root state split.
// Per depth:
//   P1  Z = S U_C^T as partial tiles over k-groups (U fragments prefetched one
//       depth earlier into registers), then the first k-steps of A S^T on the
//       same state fragments (A resident in registers).
//   P2  one wave per parent: log-softmax over its K candidates, cum, s_beta,
//       64-bit keys; the slot-0 parent's wave sorts its high words and takes
//       the W-th as the bound T (its W best children alone reach T), and the
//       least of the parents' best children is a second bound; the
//       previous level's path ranks; the rest of A S^T.
//   P3a keys with high word >= T compacted into LDS.
//   P3b survivors ranked by counting; the W smallest ranks are the level, in
//       order; this depth's staged E and h rows written into LDS.
//   P4  one wave per kept node: its state tanh(A s_parent + E[u] + h_d) split
//       into the two fp16 planes the next depth reads.
// The next depth's U fragments and E / h rows are loaded into registers one
// share per phase. After the loop: the levels to global memory, the deferred
// top-B by counting ranks over the at most L*W nodes, emission and mask.
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / kWave;
constexpr int RT = 256;            // state width
constexpr int SSTR = RT + 8;       // state-plane row stride (fp16 elements)
constexpr int ASTR = RT + 4;       // A*S row stride (floats)
constexpr int kWMax = 16;
constexpr int kLMax = 31;
static_assert(kLMax * kWMax <= kT, "the tail takes one supertree node per thread");
constexpr int kSkCap = 1024;       // survivor keys (>= 16 parents x 64 candidates)
constexpr size_t kMaxSmem = 160 * 1024;
constexpr int kMaxMergeS = 8;     // slice lists merged in the prologue

// Fixed LDS region (compile-time offsets, in bytes).
template <int KC>
struct FX {
  static constexpr int NT = KC / 16;                         // candidate tiles of Z
  static constexpr int KQ = 16 / NT > 8 ? 8 : 16 / NT;       // k-groups of Z
  static constexpr int KSQ = 8 / KQ;                         // 32-wide k-steps per group
  static constexpr int ZSTR = KC + 4;
  static constexpr int NEVEC = KC * RT / 8;                  // 16-byte vectors of E rows
  static constexpr int NEV = NEVEC >= kT ? NEVEC / kT : 1;   // per thread
  static constexpr size_t o_sh = 0;
  static constexpr size_t o_sl = o_sh + 2 * 16 * SSTR;
  static constexpr size_t o_zp = o_sl + 2 * 16 * SSTR;
  static constexpr size_t zp_bytes = 4 * KQ * 16 * ZSTR;
  static constexpr size_t sk_bytes = 8 * (kSkCap + 4);
  static constexpr size_t o_sk = o_zp;                // survivors reuse the Z partials (P3 vs P1/P2)
  static constexpr size_t o_as = o_zp + (zp_bytes > sk_bytes ? zp_bytes : sk_bytes);
  static constexpr size_t o_ec = o_as + 2 * 4 * 16 * ASTR;  // [KC][RT]
  static constexpr size_t o_hb = o_ec + 2 * KC * RT;          // [RT]
  static constexpr size_t o_ck = o_hb + 4 * RT;
  static constexpr size_t o_win = o_ck + 4 * 16 * KC;
  static constexpr size_t o_misc = o_win + 8 * 16;
  static constexpr size_t fixed = o_misc + 4 * 32;
};

// Variable LDS region (depends on L, W, B).
struct VOff {
  size_t cid, clog, tok, ps, lex, cum, sb, cnt, nkey, eix, nd, epar, total;
};

__host__ __device__ inline size_t fal16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline VOff voff(int L, int KC, int W, int B, size_t fixed) {
  VOff o{};
  size_t off = fixed;
  auto take = [&](size_t b) {
    const size_t x = off;
    off = fal16(off + b);
    return x;
  };
  const size_t LW = (size_t)L * W;
  o.cid = take(4ul * L * KC);
  o.clog = take(4ul * L * KC);
  o.tok = take(4 * LW);
  o.ps = take(4 * LW);
  o.lex = take(4 * LW);
  o.cum = take(4 * LW);
  o.sb = take(4 * LW);
  o.cnt = take(4 * 32);
  o.nkey = take(8 * (LW + 16));
  o.eix = take(4 * LW);
  o.nd = take(4 * 32);
  o.epar = take(4ul * B);
  o.total = off;
  return o;
}

size_t fixed_bytes(int KC) {
  switch (KC) {
    case 16: return FX<16>::fixed;
    case 32: return FX<32>::fixed;
    default: return FX<64>::fixed;
  }
}

struct FLay {
  LDS uint16_t* Sh;    // [16][SSTR] parent states, fp16 high part
  LDS uint16_t* Sl;    // [16][SSTR] fp16 low part (the rest of the fp32 value)
  LDS float* Zp;       // [KQ][16][ZSTR]
  LDS float* AS;       // [2][16][ASTR] A*S over the two halves of the state
  LDS uint16_t* EC;    // [KC][RT] E rows of the depth's candidates
  LDS float* hb;       // [RT] h row of the depth
  LDS float* cumK;     // [16][KC]
  LDS uint64_t* sk;    // [kSkCap + 4] survivor keys
  LDS uint64_t* win;   // [16] the depth's survivors by rank
  LDS int* misc;       // [32]: by depth parity, bounds (0, 1 and 4, 5) and survivor counts (2, 3); 16..31 level keys
  LDS int* cid;        // [L][KC]
  LDS float* clog;     // [L][KC]
  LDS int* lv_tok;     // [L][W]
  LDS int* lv_ps;
  LDS int* lv_lex;
  LDS float* lv_cum;
  LDS float* lv_sb;
  LDS int* lv_cnt;     // [32]
  LDS uint64_t* nkey;  // [L*W + 16] node keys, zero-padded
  LDS int* eix;        // [L*W] rank counters
  LDS int* nd;         // [32] selected path ranks per level
  LDS int* epar;       // [B] emitted parent index
};

template <int KC>
__device__ __forceinline__ FLay make_flay(const VOff& o) {
  using C = FX<KC>;
  extern __shared__ __align__(16) char smem[];
  LDS char* b = (LDS char*)smem;
  FLay s;
  s.Sh = (LDS uint16_t*)(b + C::o_sh);
  s.Sl = (LDS uint16_t*)(b + C::o_sl);
  s.Zp = (LDS float*)(b + C::o_zp);
  s.AS = (LDS float*)(b + C::o_as);
  s.EC = (LDS uint16_t*)(b + C::o_ec);
  s.hb = (LDS float*)(b + C::o_hb);
  s.cumK = (LDS float*)(b + C::o_ck);
  s.sk = (LDS uint64_t*)(b + C::o_sk);
  s.win = (LDS uint64_t*)(b + C::o_win);
  s.misc = (LDS int*)(b + C::o_misc);
  s.cid = (LDS int*)(b + o.cid);
  s.clog = (LDS float*)(b + o.clog);
  s.lv_tok = (LDS int*)(b + o.tok);
  s.lv_ps = (LDS int*)(b + o.ps);
  s.lv_lex = (LDS int*)(b + o.lex);
  s.lv_cum = (LDS float*)(b + o.cum);
  s.lv_sb = (LDS float*)(b + o.sb);
  s.lv_cnt = (LDS int*)(b + o.cnt);
  s.nkey = (LDS uint64_t*)(b + o.nkey);
  s.eix = (LDS int*)(b + o.eix);
  s.nd = (LDS int*)(b + o.nd);
  s.epar = (LDS int*)(b + o.epar);
  return s;
}


// Two fp16 parts of 4 consecutive fp32 state values (8 bytes per plane):
// hi = the value truncated to fp16, lo = the remainder (exact in fp32)
// truncated to fp16. |hi - s| < 2^-10 |s| and truncating the remainder loses
// less than 2^-10 of it, so |s - (hi + lo)| < max(2^-20 |s|, 2^-24) (the
// second term where the remainder falls below the fp16 normal range).
__device__ __forceinline__ void split_store4(const FLay& s, int row, int j0, const float (&v)[4]) {
  const h16x2_t h01 = pkrtz(v[0], v[1]);
  const h16x2_t h23 = pkrtz(v[2], v[3]);
  const h16x2_t l01 = pkrtz(v[0] - (float)h01.x, v[1] - (float)h01.y);
  const h16x2_t l23 = pkrtz(v[2] - (float)h23.x, v[3] - (float)h23.y);
  const int o = row * SSTR + j0;
  *reinterpret_cast<LDS u32x2_t*>(s.Sh + o) =
      u32x2_t{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
  *reinterpret_cast<LDS u32x2_t*>(s.Sl + o) =
      u32x2_t{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
}


// Path ranks of level d (1-based) from the ranks of level d-1: the order of
// (parent's path rank, token) among the level's cnt nodes. One wave.
__device__ __forceinline__ void level_lex_wave(const FLay& s, int d, int W, int cnt, const uint32_t tok,
                                               const int ps) {
  // The level's keys (parent's lexicographic rank, token) go through LDS
  // (one wave writes, then every lane reads all of them back); a lane's rank
  // is the number of smaller keys. Keys are distinct: two children of one
  // parent carry distinct tokens.
  const int lane = lane_id();
  uint32_t k2 = 0xFFFFFFFFu;
  if (lane < cnt) {
    const int lp = d == 1 ? 0 : s.lv_lex[(d - 2) * W + min(max(ps, 0), W - 1)];
    k2 = ((uint32_t)lp << 18) | (tok & 0x3FFFFu);
  }
  LDS uint32_t* kb = reinterpret_cast<LDS uint32_t*>(s.misc + 16);
  if (lane < 16) kb[lane] = k2;
  int rk = 0;
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    const u32x4_t kk = *reinterpret_cast<const LDS u32x4_t*>(kb + c);
    rk += (kk.x < k2) + (kk.y < k2) + (kk.z < k2) + (kk.w < k2);
  }
  if (lane < cnt) s.lv_lex[(d - 1) * W + lane] = rk;
}

// Sum of a per-lane count over aligned groups of G consecutive lanes (G a
// power of two <= 16, wave-uniform); every lane of a group gets the sum.
__device__ __forceinline__ uint32_t group_sum(uint32_t c, int G) {
  if (G >= 2) c += dpp<kDppXor1>(c);
  if (G >= 4) c += dpp<kDppXor2>(c);
  if (G >= 8) c += lane_xor<4>(c);
  if (G >= 16) c += lane_xor<8>(c);
  return c;
}

template <int KC, bool MARKOV>
__global__ __launch_bounds__(kT) void tree_fast_kernel(TreeArgs a) {
  using C = FX<KC>;
  const FLay s = make_flay<KC>(voff(a.L, KC, a.W, a.B, C::fixed));
  const int q = blockIdx.x, tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int L = a.L, W = a.W, B = a.B;
  // this request's width and budget (per-request values clamped to [1, W], [1, B])
  const int Wq = a.w_req ? min(max(a.w_req[q], 1), W) : W;
  const int Bq = a.b_req ? min(max(a.b_req[q], 1), B) : B;
  const size_t lw = (size_t)q * L * W;
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  // MARKOV (no A): the Markov head, whose states have no recurrence
  // (A s_parent = 0); a separate instantiation, so the full head's code is
  // untouched by the variant
  constexpr bool markov = MARKOV;
  const uint16_t* E = static_cast<const uint16_t*>(a.E);
  const uint16_t* U = static_cast<const uint16_t*>(a.U);
  const float* hq = a.h + (size_t)q * L * RT;
  const int32_t* cid_g = a.cand_ids + (size_t)q * L * KC;
  const float* clog_g = a.cand_logit + (size_t)q * L * KC;
  const bool expand = a.d0 <= a.d1;

  // ---- wave roles ------------------------------------------------------------
  // Wave w works on half hk = w / 8 of the state (k-steps 4hk..4hk+3, each 32
  // wide) and, within it, on rows 32a..32a+31 of A*S (a = w % 8, two 16-row
  // tiles with A resident in registers) and on one Z tile: candidate tile
  // a % NT over the KSQ k-steps of its k-group a / NT (waves beyond NT*KQ/2
  // per half have no Z tile). The pass over the half starts at the Z k-group,
  // so the Z steps are the first KSQ steps.
  constexpr int ZPH = C::NT * (C::KQ / 2);   // Z waves per half
  const int sub = (lane >> 4) * 8;
  const int hk = w >> 3, aw = w & 7;
  const bool zw = aw < ZPH;
  const int z_nt = aw % C::NT, z_kg = aw / C::NT;
  const int z_kq = hk * (C::KQ / 2) + z_kg;               // global k-group of the Z partial
  const int zrot = zw ? z_kg * C::KSQ : 0;                // first local k-step of the pass
  auto kstep = [&](int i) { return hk * 4 + ((i + zrot) & 3); };

  // ---- prologue ------------------------------------------------------------
  // This wave's slice lists and the root state row are loaded first; the A
  // fragments only after the merge (their 128 KB would hold the list loads
  // and the merge behind them in the memory pipeline).
  uint64_t ks[kMaxMergeS];
  u16x8_t araw[2][4];
  const bool merge_here = expand && a.lists != nullptr;
  if (merge_here && w < L) {
    const uint64_t* lst = a.lists + (size_t)(q * L + w) * a.S * KC;
#pragma unroll
    for (int sl = 0; sl < kMaxMergeS; ++sl) ks[sl] = (sl < a.S && lane < KC) ? lst[sl * KC + lane] : 0ull;
  }
  f32x4_t h0 = {0.f, 0.f, 0.f, 0.f};
  if (expand && a.d0 == 1 && tid < RT / 4) h0 = *reinterpret_cast<const f32x4_t*>(hq + tid * 4);

  if (tid < 32) s.misc[tid] = 0;
  if (tid < 32) {
    // counts of levels expanded by this launch are set by the depth loop
    int c = 0;
    if (tid < L && !(expand && tid + 1 >= a.d0 && tid + 1 <= a.d1))
      c = min(max(a.st_count[(size_t)q * L + tid], 0), W);
    s.lv_cnt[tid] = c;
  }
  for (int i = tid; i < L * W; i += kT) {
    const int d = i / W + 1;
    const bool here = expand && d >= a.d0 && d <= a.d1;
    if (!here && (a.do_select || (expand && d == a.d0 - 1))) {
      s.lv_tok[i] = a.st_tok[lw + i];
      s.lv_ps[i] = d == 1 ? 0 : a.st_parent[lw + i];
      s.lv_sb[i] = a.st_sbeta[lw + i];
      s.lv_cum[i] = a.st_cum[lw + i];
    }
  }
  int Wp = 1;
  if (merge_here) {
    // Candidates of each position: the K best of the scan's S sorted slice
    // lists, one wave per row. The lists are merged pairwise in registers:
    // the elementwise maximum of one descending list and the other reversed
    // holds the K best of both as a bitonic sequence, which six half-cleaner
    // stages sort descending. Keys are (value key << 32) | ~id, so the order
    // is value descending, id ascending. kMaxMergeS <= 8 slices.
    for (int row = w; row < L; row += kWaves) {
      if (row != w) {
        const uint64_t* lst = a.lists + (size_t)(q * L + row) * a.S * KC;
#pragma unroll
        for (int sl = 0; sl < kMaxMergeS; ++sl) ks[sl] = (sl < a.S && lane < KC) ? lst[sl * KC + lane] : 0ull;
      }
      uint32_t ah = (uint32_t)(ks[0] >> 32), al = (uint32_t)ks[0];
#pragma unroll
      for (int sl = 1; sl < kMaxMergeS; ++sl) {
        if (sl < a.S) {
          const uint32_t bh = lane_rev(ks[sl] >> 32), bl = lane_rev((uint32_t)ks[sl]);
          const bool tb = (((uint64_t)bh << 32) | bl) > (((uint64_t)ah << 32) | al);
          ah = tb ? bh : ah;
          al = tb ? bl : al;
          bitonic_stage<64, 32>(ah, al);
          bitonic_stage<64, 16>(ah, al);
          bitonic_stage<64, 8>(ah, al);
          bitonic_stage<64, 4>(ah, al);
          bitonic_stage<64, 2>(ah, al);
          bitonic_stage<64, 1>(ah, al);
        }
      }
      if (lane < KC) {
        const bool ok = (ah | al) != 0u;
        const int id = ok ? (int)(0xFFFFFFFFu - al) : -1;
        const float val = ok ? (a.lbf16 ? bf16_key_to_f32(ah) : key_to_f32(ah)) : -__builtin_huge_valf();
        s.cid[row * KC + lane] = (id < 0 || id >= a.V) ? 0 : id;
        s.clog[row * KC + lane] = val;
        a.cand_ids_out[(size_t)(q * L + row) * KC + lane] = id;
        a.cand_logit_out[(size_t)(q * L + row) * KC + lane] = val;
      }
    }
  } else if (expand) {
    for (int i = tid; i < L * KC; i += kT) {
      const int c = cid_g[i];
      s.cid[i] = (c < 0 || c >= a.V) ? 0 : c;
      s.clog[i] = clog_g[i];
    }
  }
  if (expand && a.d0 == 1 && w == 0) {
    // The root state h_0 is not bounded like the tanh states below it: it is
    // held in the fp16 planes as h_0 * 2^-t, with t the smallest shift that
    // brings max |h_0| under 2^15, and the depth-1 products it feeds (its Z
    // row and its A*s) are multiplied by 2^t again. Power-of-two scaling is
    // exact, and t = 0 leaves every value as it was.
    const float m = wave_max_f32(fmaxf(fmaxf(fabsf(h0[0]), fabsf(h0[1])), fmaxf(fabsf(h0[2]), fabsf(h0[3]))));
    const int t = m >= 32768.f ? __builtin_amdgcn_frexp_expf(m) - 15 : 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) h0[e] = __builtin_amdgcn_ldexpf(h0[e], -t);
    if (lane == 0) s.misc[8] = t;
  }
  if (expand) {
    // parents of the first expanded depth: the root (state h_0) or the stored level
    if (a.d0 > 1) Wp = min(max(a.st_count[(size_t)q * L + a.d0 - 2], 1), W);
    const float* st = a.st_state + (size_t)q * W * RT;
    for (int i = tid; i < 16 * RT / 4; i += kT) {
      const int p = i / (RT / 4), j0 = (i % (RT / 4)) * 4;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.d0 == 1 && p == 0) {
        v[0] = h0[0];
        v[1] = h0[1];
        v[2] = h0[2];
        v[3] = h0[3];
      } else if (a.d0 > 1 && p < Wp) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = st[p * RT + j0 + e];
      }
      split_store4(s, p, j0, v);
    }
  }
  // A fragments: 1 KB contiguous runs of the fp16 copy the scan launch
  // staged, or (without it) 16 rows x 16 bytes of A per load, converted below.
  // Issued after the parents' states above: their loads are conditional (a
  // launch that starts below depth 1), so the compiler waits for every
  // outstanding load where those paths join, which would include these.
  if constexpr (markov) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) araw[t][i] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  } else if (expand && a.a_frag) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        araw[t][i] = *reinterpret_cast<const u16x8_t*>(
            a.a_frag + ((size_t)((w * 2 + t) * 4 + ((i + zrot) & 3)) * kWave + lane) * 8);
  } else if (expand) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* arow = A + (size_t)(aw * 32 + t * 16 + (lane & 15)) * RT + sub;
#pragma unroll
      for (int i = 0; i < 4; ++i) araw[t][i] = *reinterpret_cast<const u16x8_t*>(arow + kstep(i) * 32);
    }
  }
  __syncthreads();

  // ---- register-resident operands and the prefetch ---------------------------
  // Every global load of the depth loop goes to registers: the compiler then
  // counts them in issue order and waits for exactly the ones a use needs
  // (loads straight into LDS would make it wait for all of them at the first
  // use of any). One share of the next depth's loads is issued per phase: a
  // wave's vector-memory issue stalls once the loads it has in flight pile
  // up. The U fragments (share i of KSQ) feed the next depth's Z tiles; the E
  // rows (share i of NEV, 16 bytes a lane) and the h row (wave 0) are written
  // into LDS one depth later, before the state update that reads them. Every
  // depth issues all shares (past the last needed depth they reload the last
  // one): with loads on every path the waits stay exact across the loop.
  h16x8_t areg[2][4];   // A fragments as fp16
  u16x8_t ureg[C::KSQ];   // U fragments (bf16) of the depth being expanded, then of the next
  u16x8_t ereg[C::NEV];   // E rows (bf16) staged for the next depth's state update
  f32x4_t hreg = {0.f, 0.f, 0.f, 0.f};   // wave 0: the h row staged with them
  auto load_u1 = [&](int d, int i) {
    if (zw) {
      const int row = s.cid[(d - 1) * KC + z_nt * 16 + (lane & 15)];
      ureg[i] = *reinterpret_cast<const u16x8_t*>(U + (size_t)row * RT + sub + kstep(i) * 32);
    }
  };
  auto load_e1 = [&](int d, int i) {
    const int v0 = w * kWave + i * kT;   // first 16-byte vector of this wave's share
    if (v0 < C::NEVEC) {
      const int v = v0 + lane;
      const int k = v / (RT / 8), c = (v % (RT / 8)) * 8;
      ereg[i] = *reinterpret_cast<const u16x8_t*>(E + (size_t)s.cid[(d - 1) * KC + k] * RT + c);
    }
    if (i == 0 && w == 0) hreg = *reinterpret_cast<const f32x4_t*>(hq + (size_t)min(d, L - 1) * RT + lane * 4);
  };
  auto store_e = [&]() {
#pragma unroll
    for (int i = 0; i < C::NEV; ++i) {
      const int v0 = w * kWave + i * kT;
      if (v0 < C::NEVEC) *reinterpret_cast<LDS u16x8_t*>(s.EC + (size_t)(v0 + lane) * 8) = ereg[i];
    }
    if (w == 0) *reinterpret_cast<LDS f32x4_t*>(s.hb + lane * 4) = hreg;
  };
  if (expand) {
#pragma unroll
    for (int i = 0; i < C::KSQ; ++i) load_u1(a.d0, i);
#pragma unroll
    for (int i = 0; i < C::NEV; ++i) load_e1(a.d0, i);
    if (a.a_frag) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) areg[t][i] = __builtin_bit_cast(h16x8_t, araw[t][i]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) areg[t][i] = bf16x8_to_f16(araw[t][i]);
    }
  }
  lds_sync();
  // 2^t of the root state's scale (1 when the launch starts below depth 1)
  const float root_scale = __builtin_amdgcn_ldexpf(1.f, s.misc[8]);

  // ---- the depth loop ----------------------------------------------------------
  for (int d = a.d0; d <= a.d1; ++d) {
    const bool need_state = d < L;
    const int par = d & 1;
    // P1: the Z tiles, then the first KSQ k-steps of this wave's A*S on the
    // same state fragments (the rest follows in P3a; the state update reads it)
    const int p16 = lane & 15;
    // Lanes of absent parents (p >= Wp) read parent 0's row: their results
    // land only in rows / columns of absent parents, which nobody reads, and
    // the loads stay branch-free.
    const int prow = p16 < Wp ? p16 : 0;
    const LDS uint16_t* rl = s.Sl + prow * SSTR + sub;
    const LDS uint16_t* rh = s.Sh + prow * SSTR + sub;
    // fp16 state fragment (low, high part) of local k-step i
    auto ld = [&](int i, h16x8_t (&dst)[2]) {
      const int o = kstep(i) * 32;
      dst[0] = *reinterpret_cast<const LDS h16x8_t*>(rl + o);
      dst[1] = *reinterpret_cast<const LDS h16x8_t*>(rh + o);
    };
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};   // A*S, two row tiles
    auto as_mfma = [&](auto ic, const h16x8_t (&fr)[2]) {
      constexpr int i = decltype(ic)::value;
      acc0 = mfma_f16(areg[0][i], fr[0], acc0);
      acc1 = mfma_f16(areg[1][i], fr[0], acc1);
      acc0 = mfma_f16(areg[0][i], fr[1], acc0);
      acc1 = mfma_f16(areg[1][i], fr[1], acc1);
    };
    // the remaining k-steps of A*S, then A*S out to LDS
    auto as_finish = [&]() {
      h16x8_t f[4 - C::KSQ][2];
#pragma unroll
      for (int i = C::KSQ; i < 4; ++i) ld(i, f[i - C::KSQ]);
      as_mfma(std::integral_constant<int, C::KSQ>{}, f[0]);
      as_mfma(std::integral_constant<int, C::KSQ + 1>{}, f[1]);
      if constexpr (C::KSQ == 1) as_mfma(std::integral_constant<int, 3>{}, f[2]);
      LDS float* asr = s.AS + (hk * 16 + p16) * ASTR + aw * 32 + (lane >> 4) * 4;
      *reinterpret_cast<LDS f32x4_t*>(asr) = acc0;
      *reinterpret_cast<LDS f32x4_t*>(asr + 16) = acc1;
    };
    {
      h16x8_t f[C::KSQ][2];
#pragma unroll
      for (int i = 0; i < C::KSQ; ++i) ld(i, f[i]);
      if (zw) {
        h16x8_t uf[C::KSQ];
#pragma unroll
        for (int i = 0; i < C::KSQ; ++i) uf[i] = bf16x8_to_f16(ureg[i]);
        f32x4_t zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < C::KSQ; ++i) {
          zacc = mfma_f16(f[i][0], uf[i], zacc);
          zacc = mfma_f16(f[i][1], uf[i], zacc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s.Zp[(z_kq * 16 + (lane >> 4) * 4 + i) * C::ZSTR + z_nt * 16 + (lane & 15)] = zacc[i];
      }
      __builtin_amdgcn_sched_barrier(0);   // the Z results go out before the A*S work is issued
      if (need_state && !markov) {
        as_mfma(std::integral_constant<int, 0>{}, f[0]);
        if constexpr (C::KSQ > 1) as_mfma(std::integral_constant<int, 1>{}, f[C::KSQ > 1 ? 1 : 0]);
      }
    }
    lds_sync();

    // P2: the parents' waves do the log-softmax and keys (the slot-0 parent's
    // wave, at raised issue priority, also the bound T: the critical path),
    // then every other wave the rest of its A*S (the slot-0 wave does its
    // share in P3b), then the first share of the next depth's U fragments
    // (the Z MFMAs of P1 were the last readers of the registers).
    const float bd = a.beta * (float)d;
    uint32_t kh = 0u, kl = 0u;
    if (w == 0) __builtin_amdgcn_s_setprio(2);
    if (w < Wp) {
      const int p = w;
      const bool v = KC == kWave ? true : lane < KC;
      const int kk = v ? lane : 0;
      float zs = 0.f;
#pragma unroll
      for (int qq = 0; qq < C::KQ; ++qq) zs += s.Zp[(qq * 16 + p) * C::ZSTR + kk];
      if (d == 1) zs *= root_scale;
      const float z = v ? zs + s.clog[(d - 1) * KC + kk] : -__builtin_huge_valf();
      const int tok = s.cid[(d - 1) * KC + kk];
      const float cp = d == 1 ? 0.f : s.lv_cum[(d - 2) * W + p];
      // exp and log on the hardware exp2/log2 (relative error about 1e-7
      // where it matters: terms near the maximum dominate the sum)
      const float m = wave_max_f32(z);
      const float ssum = wave_sum_f32(v ? __builtin_amdgcn_exp2f((z - m) * 1.4426950408889634f) : 0.f);
      const float lse = m + __builtin_amdgcn_logf(ssum) * 0.6931471805599453f;
      const float cum = cp + fminf(z - lse, 0.f);
      if (v) s.cumK[p * KC + lane] = cum;
      kh = v ? f32_key(cum + bd) : 0u;
      kl = v ? ~(((uint32_t)tok << 10) | ((uint32_t)p << 6) | (uint32_t)lane) : 0u;
      if (Wp >= Wq && lane == 0) {
        // Second bound: with at least Wq parents, each parent's best child is
        // a distinct key, so the least of those reaches the Wq-th largest.
        // The best child's key is this parent's maximum logit through the
        // same operations as the lanes' keys; the least is taken by an LDS
        // maximum of complements (the slot starts at 0 every depth).
        const uint32_t kmax = f32_key((cp + fminf(m - lse, 0.f)) + bd);
        lds_max((LDS unsigned*)&s.misc[4 + par], ~kmax);
      }
      if (p == 0) {
        // Bound T: the W-th largest high word among the children of the
        // level's first parent (the one with the best score, its W best
        // children alone reach T). K >= W children are valid.
        uint32_t sk32 = kh;
        wave_sort_desc32(sk32);
        // the cross-lane read stays outside the one-lane branch: inside it the
        // compiler may sink the sort's last stage under that lane's mask
        const int tw = (int)readlane(sk32, W - 1);
        if (lane == 0) s.misc[par] = tw;
      }
    }
    if (w == 0) __builtin_amdgcn_s_setprio(0);
    // the level before this one: its path ranks, by a wave without a parent
    // (the state update of the level, one depth ago, had no spare wave), at
    // raised issue priority too: it is the last wave to reach the barrier
    if (a.do_select && a.d0 == 1 && d >= 2 && w == kWaves - 1) {
      __builtin_amdgcn_s_setprio(2);
      uint32_t tk = 0u;
      int ps = 0;
      if (lane < Wp) {
        const uint32_t lo = ~(uint32_t)s.win[lane];
        tk = lo >> 10;
        ps = (lo >> 6) & 15;
      }
      level_lex_wave(s, d - 1, W, Wp, tk, ps);
    }
    if (need_state && !markov && w != 0) as_finish();
    if (w == kWaves - 1) __builtin_amdgcn_s_setprio(0);
    load_u1(min(d + 1, a.d1), 0);
    lds_sync();

    // P3: survivors (high word >= T) compacted, then ranked by counting
    if (w < Wp) {
      // the larger of the two bounds (both at most the Wq-th largest key)
      const uint32_t T = max((uint32_t)s.misc[par], Wp >= Wq ? ~(uint32_t)s.misc[4 + par] : 0u);
      const bool sv = lane < KC && kh >= T;
      const uint64_t bal = __ballot(sv);
      int base = 0;
      if (lane == 0) base = lds_add(&s.misc[2 + par], __popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);
      if (sv) s.sk[base + (int)mbcnt64(bal)] = ((uint64_t)kh << 32) | kl;
    }
    if (C::KSQ > 1) load_u1(min(d + 1, a.d1), 1);
    lds_sync();
    const int nk = min(Wq, Wp * KC);
    {
      // G = 2^lg threads per survivor (up to 16), as many as waves 4..15 hold
      // (wave 0 finishes its A*S meanwhile); past 768 survivors they wrap
      // around to waves 0..3. A thread's compares are a chain of dependent
      // LDS reads, so the more threads share a survivor the shorter the
      // phase: capped at eight waves the launch took 1.45 us longer.
      const int ns = min(__builtin_amdgcn_readfirstlane(s.misc[2 + par]), kSkCap);
      int lg = 4;
      while (lg > 0 && (ns << lg) > 12 * kWave) --lg;
      const int G = 1 << lg;
      const int per = (ns + G - 1) >> lg;
      const int rt = (tid + kT - 4 * kWave) & (kT - 1);
      const int x = rt >> lg, seg = rt & (G - 1);
      uint64_t kx = 0ull;
      uint32_t cnt = 0u;
      const bool wave_ranks = (rt & ~(kWave - 1)) < (ns << lg);   // other waves hold no survivor's group
      if (wave_ranks && x < ns) {
        kx = s.sk[x];
        const int y0 = seg * per, y1 = min(ns, y0 + per);
        for (int y = y0; y < y1; y += 4) {
          uint64_t k4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) k4[e] = s.sk[y + e];
#pragma unroll
          for (int e = 0; e < 4; ++e) cnt += (y + e < y1 && k4[e] > kx) ? 1u : 0u;
        }
      }
      const int rk = wave_ranks ? (int)group_sum(cnt, G) : W;
      if (x < ns && seg == 0 && rk < Wq) {
        const uint32_t lo = ~(uint32_t)kx;
        const int k = lo & 63, p = (lo >> 6) & 15;
        const int row = (d - 1) * W + rk;
        const float cum = s.cumK[p * KC + k];
        s.win[rk] = kx;
        s.lv_tok[row] = (int)(lo >> 10);
        s.lv_ps[row] = p;
        s.lv_cum[row] = cum;
        s.lv_sb[row] = cum + bd;
      }
      if (tid == 0) s.lv_cnt[d - 1] = nk;
      // the other parity's bounds and count are free again (read one depth ago)
      if (tid < 3) s.misc[(par ^ 1) + 2 * tid] = 0;
    }
    if (need_state && !markov && w == 0) as_finish();
    // this depth's staged E/h rows into LDS, then the next depth's first E share
    store_e();
    load_e1(min(d + 1, L), 0);
    lds_sync();

    // P4: states of the survivors, one wave each; path ranks of the level
    if (need_state && w < nk) {
      const uint32_t lo = ~(uint32_t)s.win[w];
      const int k = lo & 63, p = (lo >> 6) & 15;
      const int j0 = lane * 4;
      f32x4_t as4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!markov) {
        const f32x4_t a0 = *reinterpret_cast<const LDS f32x4_t*>(s.AS + p * ASTR + j0);
        const f32x4_t a1 = *reinterpret_cast<const LDS f32x4_t*>(s.AS + (16 + p) * ASTR + j0);
        as4 = a0 + a1;
        if (d == 1) as4 *= root_scale;
      }
      const u32x2_t e2 = *reinterpret_cast<const LDS u32x2_t*>(s.EC + (size_t)k * RT + j0);
      const f32x4_t h4 = *reinterpret_cast<const LDS f32x4_t*>(s.hb + j0);
      const float ev[4] = {bf16_to_f32(e2.x & 0xFFFFu), bf16_to_f32(e2.x >> 16), bf16_to_f32(e2.y & 0xFFFFu),
                           bf16_to_f32(e2.y >> 16)};
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = tanh_fast((as4[i] + ev[i]) + h4[i]);
      split_store4(s, w, j0, v);
      if (d == a.d1)
        *reinterpret_cast<f32x4_t*>(a.st_state + ((size_t)q * W + w) * RT + j0) = f32x4_t{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int i = 1; i < C::NEV; ++i) load_e1(min(d + 1, L), i);
    if (a.do_select && a.d0 == 1 && d == a.d1 && w == kWaves - 1) {
      uint32_t tk = 0u;
      int ps = 0;
      if (lane < nk) {
        const uint32_t lo = ~(uint32_t)s.win[lane];
        tk = lo >> 10;
        ps = (lo >> 6) & 15;
      }
      level_lex_wave(s, d, W, nk, tk, ps);
    }
    Wp = nk;
    lds_sync();
  }
  vmcnt_zero();   // the last depth's loads for a following one (unused) land before LDS is reused
  __syncthreads();

  // ---- the expanded levels to global memory ---------------------------------------
  if (expand) {
    const int n0 = (a.d0 - 1) * W, n1 = a.d1 * W;
    // stored by the upper half of the workgroup while the lower half builds
    // the node keys of the selection below
    for (int i = n0 + ((tid + kT / 2) & (kT - 1)); i < n1; i += kT) {
      const int d = i / W + 1, sl = i - (d - 1) * W;
      if (sl < s.lv_cnt[d - 1]) {
        a.st_tok[lw + i] = s.lv_tok[i];
        a.st_parent[lw + i] = d == 1 ? 0 : s.lv_ps[i];
        a.st_cum[lw + i] = s.lv_cum[i];
        a.st_sbeta[lw + i] = s.lv_sb[i];
      } else {
        a.st_tok[lw + i] = -1;
        a.st_parent[lw + i] = -1;
        a.st_cum[lw + i] = -__builtin_huge_valf();
        a.st_sbeta[lw + i] = -__builtin_huge_valf();
      }
    }
    for (int d = a.d0 + tid; d <= a.d1; d += kT) a.st_count[(size_t)q * L + d - 1] = s.lv_cnt[d - 1];
  }
  if (!a.do_select) return;

  // ---- deferred global top-B -----------------------------------------------------
  if (!(expand && a.d0 == 1)) {
    if (w == 0) {
      for (int d = 1; d <= L; ++d) {
        const int cnt = s.lv_cnt[d - 1];
        uint32_t tk = 0u;
        int ps = 0;
        if (lane < cnt) {
          tk = (uint32_t)s.lv_tok[(d - 1) * W + lane];
          ps = s.lv_ps[(d - 1) * W + lane];
        }
        level_lex_wave(s, d, W, cnt, tk, ps);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  // Node keys (0 for empty slots), zero-padded to a multiple of 16; the rank
  // counters start at 0. The level arrays are read whole, in one round trip.
  const int N = L * W, N16 = (N + 15) & ~15;
  for (int i = tid; i < N16; i += kT) {
    uint64_t key = 0ull;
    if (i < N) {
      const int d = i / W + 1, sl = i - (d - 1) * W;
      const int cnt = s.lv_cnt[d - 1];
      const uint32_t tok = (uint32_t)s.lv_tok[i] & 0x3FFFFu;
      const uint32_t ps = d == 1 ? 0u : ((uint32_t)s.lv_ps[i] & 0x1FFu);
      const uint32_t kv = f32_key(s.lv_sb[i]);
      if (sl < cnt) key = ((uint64_t)kv << 32) | (uint64_t)(0xFFFFFFFFu - (((uint32_t)d << 27) | (tok << 9) | ps));
      s.eix[i] = 0;
    }
    s.nkey[i] = key;
  }
  if (tid < 32) s.nd[tid] = 0;   // per level: bit (path rank) set when the node is selected
  lds_sync();
  {
    // Rank of each node = the number of larger keys. Nodes go one per lane
    // over NW waves, the keys over G = 16 / NW segments, one per group of NW
    // waves: all lanes of a wave compare against the same keys, read by
    // broadcast, and the partial counts are added in LDS.
    const int NW = (N16 + kWave - 1) / kWave;
    const int G = kWaves / NW;
    const int seg = w / NW, x = (w - seg * NW) * kWave + lane;
    if (seg < G) {
      const uint64_t kx = x < N16 ? s.nkey[x] : ~0ull;
      const int KS = (((N16 + G - 1) / G) + 15) & ~15;   // keys per segment, a multiple of 16
      const int y0 = seg * KS, y1 = min(N16, y0 + KS);
      uint32_t c = 0u;
      for (int y = y0; y < y1; y += 16) {   // eight 16-byte reads in flight per step
        u64x2_t k2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) k2[e] = *reinterpret_cast<const LDS u64x2_t*>(s.nkey + y + 2 * e);
#pragma unroll
        for (int e = 0; e < 8; ++e) c += (k2[e].x > kx ? 1u : 0u) + (k2[e].y > kx ? 1u : 0u);
      }
      if (x < N && c) lds_add(&s.eix[x], (int)c);
    }
  }
  lds_sync();
  // a node is selected when its rank is below B_q (empty slots: key 0, never)
  for (int i = tid; i < N; i += kT)
    if (s.nkey[i] != 0ull && s.eix[i] < Bq) lds_or(&s.nd[i / W], 1 << s.lv_lex[i]);
  lds_sync();
  // Emitted index: selected nodes of earlier levels, then selected nodes of
  // the level with a smaller path rank (breadth-first order = path order).
  // Every thread totals the selection. A node's parent index comes from the
  // same per-level bits: the parent of a selected node is selected (prefix
  // closure), at the parent level's base plus its rank among that level's
  // selected path ranks. One node per thread (L * W <= 1024).
  int n = 0, base = 0, basep = 0;
  const int d_i = min(tid / W + 1, L);
#pragma unroll
  for (int j = 0; j < 32; j += 4) {
    const u32x4_t v4 = *reinterpret_cast<const LDS u32x4_t*>(s.nd + j);
    const int p[4] = {(int)__popc(v4.x), (int)__popc(v4.y), (int)__popc(v4.z), (int)__popc(v4.w)};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      n += p[t];
      base += j + t < d_i - 1 ? p[t] : 0;
      basep += j + t < d_i - 2 ? p[t] : 0;
    }
  }
  int32_t* o_tok = a.tok + (size_t)q * B;
  int32_t* o_dep = a.depth + (size_t)q * B;
  int32_t* o_par = a.parent + (size_t)q * B;
  float* o_sc = a.score + (size_t)q * B;
  int32_t* o_slot = a.slot + (size_t)q * B;
  if (tid < N) {
    const int i = tid, d = d_i, sl = i - (d - 1) * W;
    const uint32_t m = (uint32_t)s.nd[d - 1], mp = d > 1 ? (uint32_t)s.nd[d - 2] : 0u;
    const int lx = s.lv_lex[i];
    const int psl = min(max(s.lv_ps[i], 0), W - 1);
    const bool sel = s.nkey[i] != 0ull && ((m >> lx) & 1u);
    const int tk = s.lv_tok[i];
    const float sb = s.lv_sb[i];
    if (sel) {
      const int e = base + __popc(m & ((1u << lx) - 1u));
      int pe = -1;
      if (d > 1) {
        const int plx = s.lv_lex[(d - 2) * W + psl];
        pe = ((mp >> plx) & 1u) ? basep + __popc(mp & ((1u << plx) - 1u)) : -1;
      }
      o_tok[e] = tk;
      o_dep[e] = d;
      o_par[e] = pe;
      o_sc[e] = sb;
      o_slot[e] = sl;
      s.epar[e] = pe;
    }
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
  lds_sync();

  // ---- ancestor mask ------------------------------------------------------------------
  const int words = (B + 63) / 64;
  uint64_t* mq = a.mask + (size_t)q * B * words;
  if (words == 1) {
    // one wave, pointer doubling with lane shuffles: after round k, mb covers
    // a node and its 2^k - 1 nearest ancestors and an is its 2^k-th ancestor
    if (w == 0) {
      int an = lane < n ? s.epar[lane] : -1;
      uint64_t mb = lane < n ? (1ull << lane) : 0ull;
      for (int span = 1; span < L; span *= 2) {
        const int src = (an >= 0 && an < lane) ? an : lane;
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)mb, src, kWave);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(mb >> 32), src, kWave);
        const int an2 = __shfl(an, src, kWave);
        if (src != lane) {
          mb |= ((uint64_t)hi << 32) | lo;
          an = an2;
        } else {
          an = -1;
        }
      }
      if (lane < B) mq[lane] = mb;
    }
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

}  // namespace

TreePlan tree_fast_plan(const TreeArgs& a) {
  TreePlan p{};
  p.ok = false;
  const bool al = ((((uintptr_t)a.A) | ((uintptr_t)a.E) | ((uintptr_t)a.U) | ((uintptr_t)a.h) |
                    ((uintptr_t)a.st_state)) & 15u) == 0;
  if (a.exact || !a.bf16 || a.r != RT || !(a.K == 16 || a.K == 32 || a.K == 64) || a.W > kWMax || a.W < 1 || a.V < a.K ||
      a.L > kLMax || a.B > 1024 || !al || (a.lists && a.S > kMaxMergeS))
    return p;
  p.mode = 3;
  p.kq = 16 / (a.K / 16) > 8 ? 8 : 16 / (a.K / 16);
  p.smem = voff(a.L, a.K, a.W, a.B, fixed_bytes(a.K)).total;
  p.ok = p.smem <= kMaxSmem;
  return p;
}

hipError_t launch_tree_fast(const TreePlan& p, const TreeArgs& a, hipStream_t s) {
  dim3 grid(a.n_req), block(kT);
  hipError_t e = hipSuccess;
#define DT_FAST(KCV, MK)                                                                                      \
  do {                                                                                                        \
    e = hipFuncSetAttribute((const void*)tree_fast_kernel<KCV, MK>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                            (int)p.smem);                                                                     \
    if (e != hipSuccess) return e;                                                                            \
    hipLaunchKernelGGL((tree_fast_kernel<KCV, MK>), grid, block, p.smem, s, a);                              \
  } while (0)
  const bool mk = a.A == nullptr;   // the Markov head
  if (a.K == 16) {
    if (mk) DT_FAST(16, true);
    else DT_FAST(16, false);
  } else if (a.K == 32) {
    if (mk) DT_FAST(32, true);
    else DT_FAST(32, false);
  } else {
    if (mk) DT_FAST(64, true);
    else DT_FAST(64, false);
  }
#undef DT_FAST
  return hipGetLastError();
}

}  // namespace dartree
