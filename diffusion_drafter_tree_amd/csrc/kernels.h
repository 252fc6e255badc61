// Host-side launchers of the gfx950 kernels (internal to libdartree).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dartree {

// ---- steps a1 (+ a0 in the same launch) -----------------------------------
struct ScanArgs {
  const void* logits;   // [rows][V]
  int rows, V, K;
  int S, slice, n_scan;  // filled from the plan
  uint64_t* lists;      // [rows][S][K] when S > 1
  int32_t* cand_ids;    // [rows][K] when S == 1
  float* cand_logit;
  // head projection tiles (bf16 MFMA path), n_head = 0 for none
  const uint16_t* H;    // [M][D]
  const uint16_t* Pt;   // [r][D]
  float* h;             // [M][r]
  int M, D, r, n_head;
  int head_big;         // wide launch only: 64 x 64 head tiles (head_big_ok)
  // staging of A (bf16 [256][256]) as fp16 MFMA fragments for the
  // block-decoding tree kernel: n_afrag = 16 workgroups (one per tree wave)
  // write a_frag[wave][tile][k-step][lane][8], 0 for none
  const uint16_t* A;
  uint16_t* a_frag;
  int n_afrag;
  // words zeroed by the launch (the split tree kernel's flags), 0 for none
  uint32_t* clear;
  int n_clear;
};
constexpr int kAFragWaves = 16;                        // tree waves holding A fragments
constexpr size_t kAFragBytes = (size_t)256 * 256 * 2;  // one fp16 copy of A
struct ScanPlan {
  int S, slice, nv, n_scan, merge_ept;
  size_t list_bytes;
  bool wide;   // K > 64: the wide selection (histogram-ordered survivors)
  bool ok;
};
ScanPlan scan_plan(int rows, int V, int K, bool bf16);
bool head_mfma_ok(bool bf16, const void* H, const void* Pt, int D, int r);
// 64 x 64 head tiles staged through LDS: many rows, r % 64 == 0, D % 512 == 0
bool head_big_ok(int M, int D, int r);
int head_tiles(bool big, int M, int r);
hipError_t launch_scan(const ScanPlan& p, bool bf16, const ScanArgs& a, hipStream_t s);
hipError_t launch_merge(const ScanPlan& p, int rows, int K, bool bf16, const uint64_t* lists, int32_t* cand_ids,
                        float* cand_logit, hipStream_t s);
hipError_t launch_head_valu(bool bf16, const void* H, const void* Pt, float* h, int M, int D, int r, hipStream_t s);
// h = P^T H on its own (bf16 MFMA tiles when possible, else fp32 FMAs)
hipError_t launch_head(bool bf16, const void* H, const void* Pt, float* h, int M, int D, int r, hipStream_t s);

// ---- steps a2..a5 in one workgroup per request -------------------------------
struct TreeArgs {
  int n_req, L, V, K, W, B, r;
  float beta;
  bool bf16;
  bool exact;                 // the head asks for the exact (split-bf16) general kernel
  const void* A;
  const void* E;
  const void* U;
  const int32_t* cand_ids;    // [n][L][K]
  const float* cand_logit;    // [n][L][K]
  // when set (block-decoding kernel only): the scan's S sorted slice lists
  // [n][L][S][K] of 64-bit keys; the kernel merges them into the candidates
  // and writes cand_ids / cand_logit itself
  const uint64_t* lists;
  // when set (block-decoding kernel only): A as fp16 fragments staged by the
  // scan launch (layout of ScanArgs::a_frag); otherwise loaded from A
  const uint16_t* a_frag;
  int32_t* cand_ids_out;      // written with the merged candidates
  float* cand_logit_out;
  int S;
  bool lbf16;                 // logits were bf16 (key width of the lists)
  const float* h;             // [n][L][r]
  int32_t* st_tok;            // [n][L][W]
  int32_t* st_parent;         // [n][L][W]
  float* st_cum;              // [n][L][W]
  float* st_sbeta;            // [n][L][W]
  int32_t* st_count;          // [n][L]
  const int32_t* w_req;       // [n] per-request width, or null (W for all)
  const int32_t* b_req;       // [n] per-request budget, or null (B for all)
  float* st_state;            // [n][W][r]
  int d0, d1;                 // depths to expand (d1 < d0: none)
  bool do_select, do_mask;
  int32_t* n_sel;             // [n]
  int32_t* tok;               // [n][B]
  int32_t* depth;             // [n][B]
  int32_t* parent;            // [n][B]
  float* score;               // [n][B]
  int32_t* slot;              // [n][B]
  uint64_t* mask;             // [n][B][ceil(B/64)]
  // general MFMA kernel only: a request over `split` workgroups (1: one),
  // exchanging contraction slices through xch [n][L][W][ceil16(K) + r] and the
  // per-depth flags xflag [n][split][L] (zero at launch)
  int split;
  float* xch;
  uint32_t* xflag;
  uint32_t split_wait;        // longest wait for another part's slice, in 10 ns ticks
};
struct TreePlan {
  int mode;          // 0 VALU, 1 MFMA general, 2 MFMA resident/prefetched, 3 block-decoding kernel
  int kq;            // k-groups of the score contraction (mode 2)
  bool planes;       // mode 1: parents' states held as split bf16 planes
  int split;         // mode 1: workgroups per request
  size_t smem;       // dynamic LDS bytes
  bool ok;
};
// mode 3 (tree_fast.hip) when the shapes allow it, else the general kernel
TreePlan tree_plan(const TreeArgs& a);
hipError_t launch_tree(const TreePlan& p, const TreeArgs& a, hipStream_t s);
TreePlan tree_fast_plan(const TreeArgs& a);
hipError_t launch_tree_fast(const TreePlan& p, const TreeArgs& a, hipStream_t s);

hipError_t launch_mask(int n_req, int B, const int32_t* n_sel, const int32_t* parent, uint64_t* mask, hipStream_t s);

// ---- the drafter's LM head fused with the top-K (the step before a1) ---------
struct LmheadPlan {
  int S;           // vocabulary slabs (workgroups per 16 rows)
  int ntiles;      // 16-column tiles of the vocabulary
  int slab_cols;   // columns of the widest slab
  int kc;          // D chunk staged in LDS
  int ring;        // k-steps of head loads in flight a wave
  size_t smem, list_bytes;
  bool ok;
};
// bf16 X [rows][D] and Wlm [V][D]; K <= 64, D a multiple of 256
LmheadPlan lmhead_plan(int rows, int V, int D, int K);
hipError_t launch_lmhead_topk(const LmheadPlan& p, const uint16_t* X, const uint16_t* Wlm, int rows, int V, int D,
                              int K, uint64_t* lists, int32_t* cand_ids, float* cand_logit, hipStream_t s);

// measurement utility: one read of bytes (a multiple of 16) at buf
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

// ---- heap-serial construction (the "pop then correct" baseline) -------------
constexpr int kSerialMaxB = 511;   // pop indices pack into 9 bits of the node key
struct SerialArgs {
  int n_req, L, V, K, B, r;
  float beta;
  const void* A;
  const void* E;
  const void* U;
  const int32_t* cand_ids;    // [n][L][K]
  const float* cand_logit;    // [n][L][K]
  const float* h;             // [n][L][r]
  float* states;              // [n][B + 1][r] workspace
  int32_t* n_sel;             // [n]
  int32_t* tok;               // [n][B], pop order
  int32_t* depth;             // [n][B]
  int32_t* parent;            // [n][B]: pop index of the parent, -1 for the root
  float* score;               // [n][B]: s_beta
};
hipError_t launch_serial(const SerialArgs& a, bool bf16w, hipStream_t s);

// ---- verification consumer with a synthetic target -----------------------------
struct VerifyArgs {
  int n_req, L, B, dh;
  const int32_t* n_sel;       // [n]
  const int32_t* tok;         // [n][B] emitted tree
  const int32_t* depth;       // [n][B]
  const int32_t* parent;      // [n][B]
  const uint64_t* mask;       // [n][B][ceil(B/64)]
  const int32_t* target;      // [n][L]
  const float* Q;             // [n][B][dh]
  const float* K;
  const float* V;
  int32_t* acc_len;           // [n]
  int32_t* acc_nodes;         // [n][L]
  float* out;                 // [n][B][dh]
};
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);
hipError_t launch_fill_u32(void* p, size_t n_words, uint32_t value, hipStream_t s);

// bf16 head weights beyond fp16's range (magnitude >= 2^16): *flags gets
// bit 0 for A (r x r, may be null), bit 1 for U (V x r)
hipError_t launch_head_check(const uint16_t* A, const uint16_t* U, int V, int r, int32_t* flags, hipStream_t s);

}  // namespace dartree
