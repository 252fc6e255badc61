// Host-side launchers of the gfx950 kernels (internal to libdartree).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dartree {

// ---- step a1: top-K candidates --------------------------------------------
struct TopkPlan {
  int nv;            // 16-byte vectors per thread in the chunk pass
  int chunks;        // chunks per row
  int chunk_elems;   // elements per chunk
  int merge_ept;     // keys per thread in the per-row merge
  int grid;          // workgroups
  size_t list_bytes;    // per-chunk top-K lists (workspace)
  size_t ticket_bytes;  // per-row tickets (workspace, zero between calls)
};
TopkPlan topk_plan(int rows, int V, int K, bool bf16);
hipError_t launch_topk(const TopkPlan& p, bool bf16, const void* logits, int V, int K, uint64_t* lists,
                       unsigned int* tickets, int32_t* cand_ids, float* cand_logit, hipStream_t s);

// ---- step a0: head inputs h = P^T H ----------------------------------------
hipError_t launch_head_states(bool bf16, const void* H, const void* Pt, float* h, int M, int D, int r, hipStream_t s);

// ---- steps a2 + a3: depth-by-depth expansion --------------------------------
struct ExpandArgs {
  int n_req, L, V, K, W, r;
  float beta;
  bool bf16;
  const void* A;
  const void* E;
  const void* U;
  const int32_t* cand_ids;    // [n][L][K]
  const float* cand_logit;    // [n][L][K]
  const float* h;             // [n][L][r]
  int32_t* st_tok;            // [n][L][W]
  int32_t* st_parent;         // [n][L][W]
  float* st_cum;              // [n][L][W]
  float* st_sbeta;            // [n][L][W]
  int32_t* st_count;          // [n][L]
  float* st_state;            // [n][W][r]
  int d0, d1;
};
size_t expand_smem_bytes(int K, int W, int r);
hipError_t launch_expand(const ExpandArgs& a, hipStream_t s);

// ---- step a4 + a5: global top-B, breadth-first emission, mask ---------------
struct SelectArgs {
  int n_req, L, W, B;
  const int32_t* st_tok;
  const int32_t* st_parent;
  const float* st_sbeta;
  const int32_t* st_count;
  int32_t* n_sel;   // [n]
  int32_t* tok;     // [n][B]
  int32_t* depth;   // [n][B]
  int32_t* parent;  // [n][B]
  float* score;     // [n][B]
  int32_t* slot;    // [n][B]
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_mask(int n_req, int B, const int32_t* n_sel, const int32_t* parent, uint64_t* mask, hipStream_t s);

hipError_t launch_fill_u32(void* p, size_t n_words, uint32_t value, hipStream_t s);

}  // namespace dartree
