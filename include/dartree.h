/*
 * dartree.h — C ABI of the MI355X (gfx950) draft-tree construction round.
 *
 * The method is DARTree's tree construction for a diffusion block drafter
 * (marsggbo blog "DARTree: give a diffusion drafter an AR tree", sections
 * 3.1-3.2; AINews summary "DARTree builds trees in batches before pruning").
 * One round takes the drafter's base logits and shared representations for a
 * block of L positions and produces a draft tree of at most B nodes that a
 * target model verifies in one tree-attention pass:
 *
 *   a0  h_d = P^T H_d                        dartree_head_states
 *   a1  top-K candidates per position        dartree_topk_candidates
 *   a2  batched correction scoring per depth dartree_expand_depth
 *   a3  s_beta and per-depth top-W           (same call)
 *   a4  deferred global top-B                dartree_select_topB
 *   a5  parent pointers + ancestor mask      dartree_select_topB, dartree_tree_mask
 *   all of the above in one launch           dartree_build_round
 *
 * Conventions (every call):
 *   - Every array argument is a DEVICE pointer allocated by the caller, row
 *     major and contiguous, 16-byte aligned. The library never allocates,
 *     frees or copies to the host (dartree_workspace_size tells the caller
 *     how much scratch to allocate).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Each
 *     call validates its arguments on the host, then enqueues its kernels and
 *     returns without synchronising. Results are valid once the stream
 *     reaches that point.
 *   - On any error nothing is enqueued and outputs are untouched; the status
 *     says why and dartree_last_error() (thread-local) gives detail.
 *   - Device-side faults surface at the caller's next synchronisation.
 *   - Calls are re-entrant; concurrent calls must use distinct workspaces and
 *     distinct outputs.
 *   - bf16 data is passed as raw 16-bit patterns.
 *
 * Scores (marsggbo blog, section 3.1, the score equation):
 *   s_beta(u_1..u_d) = sum_{i<=d} log q_i(u_i) + beta * d,   beta <= 0,
 * q_i is the corrected probability of the token among the K candidates of
 * position i. One comparator orders nodes everywhere: s_beta descending, then
 * depth ascending, then token id ascending, then the parent's rank (its slot
 * in its level) ascending.
 */
#ifndef DARTREE_H
#define DARTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DARTREE_OK = 0,
  DARTREE_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, beta > 0, depth out of order */
  DARTREE_ERR_UNSUPPORTED = 2,      /* beyond the implementation limits below, unknown dtype */
  DARTREE_ERR_WORKSPACE_TOO_SMALL = 3,
  DARTREE_ERR_HIP = 4               /* a HIP call failed; detail in dartree_last_error() */
} dartree_status;

typedef enum { DARTREE_F32 = 0, DARTREE_BF16 = 1 } dartree_dtype;

/* Problem sizes.
 *   n_req  requests batched in one call (>= 1)
 *   L      block length = tree depth (1..31)
 *   V      vocabulary size (K..262144)
 *   K      candidates per position (1..1024), marsggbo section 3.1 (default 64)
 *   W      nodes kept per depth (1..64), marsggbo section 3.1 (12 or 4)
 *   B      verification-tree budget (1..1024), marsggbo section 3.1 (64)
 *   r      head rank (1..1024); W*r <= 8192 and W*K <= 8192
 *   D      drafter hidden size for dartree_head_states (0 = h supplied directly)
 *   beta   depth term of s_beta; must be finite and <= 0 (Lemma 1)
 *   logits_dtype, weight_dtype: dartree_dtype of the base logits and of the
 *          head weights (A, E, U, Pt) and H. */
typedef struct {
  int32_t n_req, L, V, K, W, B, r, D;
  float beta;
  int32_t logits_dtype;
  int32_t weight_dtype;
} dartree_dims;

/* Correction head (a declared low-rank stand-in; the pages do not define the
 * head's architecture). Row-major, weight_dtype:
 *   A  [r][r]  state transition, (A s)[j] = sum_m A[j][m] s[m]
 *   E  [V][r]  token embeddings
 *   U  [V][r]  output rows: corrected logit z_c = Lbase[c] + <s_parent, U[c]>
 *   Pt [r][D]  input projection stored output-major, Pt[j][i] = P[i][j]
 *              (may be NULL when D == 0)
 * Child state: s = tanh(A s_parent + E[u] + h_d); the root state is h_0.
 * A may be NULL: the Markov-head variant (marsggbo blog section 4.3, Table 3:
 * DSpark's Markov head put in place of the correction head; the distribution
 * over a node's children is conditioned on that node's token alone). It is the head with A = 0, so a
 * state is tanh(E[u] + h_d), a function of the node's token and depth; the
 * kernels then skip the A s_parent contraction and the scan launch stages no
 * A fragments (dartree_round_plan counts those 16 workgroups regardless).
 *
 * flags: 0, or DARTREE_HEAD_EXACT. Precondition of the block-decoding tree
 * kernel (bf16 weights, r = 256, K in {16, 32, 64}, W <= 16; see
 * dartree_round_plan): it multiplies A and U in fp16, so every entry of A and
 * U must have magnitude below 2^16 (fp16's range; entries below 2^-17 are
 * truncated by at most 2^-25). dartree_head_check finds entries beyond it; a
 * head that has any must carry DARTREE_HEAD_EXACT, which sends every call to
 * the general kernel (three-part bf16 states, exact products, fp32
 * accumulation) at its cost. The root state h_0 needs no such care (it is
 * rescaled by a power of two inside the kernel). */
#define DARTREE_HEAD_EXACT 1
typedef struct {
  const void* A;
  const void* E;
  const void* U;
  const void* Pt;
  int32_t flags;
} dartree_head;

/* Range check of a bf16 head for the block-decoding kernel (see dartree_head):
 * enqueues a scan of A (r x r; skipped when NULL) and U (V x r) that writes
 * *flags (one int32 in device memory) = bit 0 when some entry of A, bit 1
 * when some entry of U has magnitude >= 2^16 (or is not finite); 0 means the
 * head meets the precondition. Reads 2 r (V + r) bytes; meant for once per
 * head, not per round. fp32 heads (weight_dtype DARTREE_F32) always give 0.
 * Errors as for the other calls. */
dartree_status dartree_head_check(const dartree_dims* dims, const dartree_head* head, int32_t* flags, void* stream);

/* The supertree: W slots per depth, kept in rank order (slot 0 best).
 *   tok         [n][L][W] int32  token id (pad -1)
 *   parent_slot [n][L][W] int32  slot of the parent in depth d-1 (depth 1: 0)
 *   cum         [n][L][W] float  sum of log q along the path (pad -inf)
 *   sbeta       [n][L][W] float  cum + beta * d (pad -inf)
 *   count       [n][L]    int32  kept nodes per depth
 *   state       [n][W][r] float  head states of the deepest expanded level,
 *                                read back by the next dartree_expand_depth
 *   next_depth  HOST field: the next depth dartree_expand_depth expects; set
 *               it to 1 before a round; each successful call advances it.
 *   width       [n] int32 or NULL: per-request width W_q of every depth (the
 *               serving knob of the blog's section 3.1, "fixed width per
 *               depth", chosen per request inside one batch); NULL means
 *               dims->W for every request. Read on the device by
 *               dartree_expand_depth and dartree_build_round; values are
 *               clamped to [1, dims->W]. Slots >= W_q are padding.
 *   budget      [n] int32 or NULL: per-request node budget B_q of the
 *               deferred top-B (the verification-tree size); NULL means
 *               dims->B. Read on the device by dartree_select_topB and
 *               dartree_build_round; values are clamped to [1, dims->B].
 *               Outputs keep their [n][B] stride; entries >= n_sel are
 *               padding as usual.
 * Memory for a per-request width or budget is the caller's and must hold its
 * values until the stream has run the call. */
typedef struct {
  int32_t* tok;
  int32_t* parent_slot;
  float* cum;
  float* sbeta;
  int32_t* count;
  float* state;
  int32_t next_depth;
  const int32_t* width;
  const int32_t* budget;
} dartree_supertree;

/* Human-readable status name; never NULL. */
const char* dartree_status_string(dartree_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* dartree_last_error(void);
/* ABI version of this library. */
int32_t dartree_version(void);

/* Scratch needed by dartree_topk_candidates and dartree_build_round for
 * these dims (bytes): the top-K's sorted slice lists, for bf16 weights of rank
 * 256 an fp16 copy of A, and, when the general tree kernel spreads a request
 * over several workgroups (dartree_round_info.tree_parts > 1), the area
 * through which they exchange each depth's contraction slices, with their
 * flags. Calls that overlap in time must use different workspaces. */
dartree_status dartree_workspace_size(const dartree_dims* dims, size_t* bytes);

/* Prepare a workspace for these dims. The current kernels keep no state in
 * the workspace between calls, so this only validates; calling it once per
 * allocation keeps callers correct should a future layout need set-up. */
dartree_status dartree_workspace_init(const dartree_dims* dims, void* ws, size_t ws_bytes, void* stream);

/* Step a0 (synthetic head input; marsggbo section 3.1: one block-parallel
 * drafter forward gives the shared representations H_d): for every request
 * and position, h[n][L][r] = P^T H[n][L][D], with Pt = P^T as in
 * dartree_head. H and Pt use weight_dtype; h is fp32. Requires D >= 1. */
dartree_status dartree_head_states(const dartree_dims* dims, const void* H, const void* Pt, float* h,
                                   void* stream);

/* Step a1 (marsggbo section 3.1, candidate generation; AINews: the 64 best
 * candidates per position): for each of the n*L rows of logits[n][L][V]
 * (logits_dtype; row i holds depth i+1), the K largest values ordered by value
 * descending, ties by token id ascending (values compare numerically, so -0 ==
 * +0). Outputs cand_ids[n][L][K] int32 and cand_logit[n][L][K] fp32 (the exact
 * widened logit). Needs a workspace of dartree_workspace_size bytes that was
 * prepared once by dartree_workspace_init. Logits must be finite. */
dartree_status dartree_topk_candidates(const dartree_dims* dims, const void* logits, int32_t* cand_ids,
                                       float* cand_logit, void* ws, size_t ws_bytes, void* stream);

/* The step before a1, fused with it (marsggbo section 3.1, basic flow: one
 * block-parallel forward of the diffusion drafter gives the block's base
 * logits, whose K best tokens per position are the candidates): for each of
 * the n*L rows of X[n][L][D] (the block's final hidden states, bf16), the base
 * logits logits[v] = sum_j X[j] * Wlm[v][j] of a drafter LM head Wlm[V][D]
 * (bf16; products exact, fp32 accumulation) and their K best, written as
 * cand_ids[n][L][K] int32 / cand_logit[n][L][K] fp32 in the order of
 * dartree_topk_candidates (value descending, ties by token id ascending). The
 * logits themselves are never written to memory. Uses dims n_req, L, V, K, D
 * and weight_dtype (must be DARTREE_BF16; UNSUPPORTED otherwise); limits
 * K <= 64, D >= 256 and a multiple of 256 (UNSUPPORTED otherwise). ws is a
 * device workspace of dartree_lmhead_workspace_size bytes (256-byte aligned),
 * overwritten. The fp32 accumulation order is the kernel's: a logit within
 * its rounding of the K-th may fall on either side of the cut. */
dartree_status dartree_lmhead_workspace_size(const dartree_dims* dims, size_t* bytes);
dartree_status dartree_lmhead_topk(const dartree_dims* dims, const void* X, const void* Wlm, int32_t* cand_ids,
                                   float* cand_logit, void* ws, size_t ws_bytes, void* stream);

/* Steps a2 + a3 (marsggbo section 3.1, depth-by-depth expansion and the score
 * equation; AINews: one batched head call per depth): expands depths
 * depth_begin..depth_end (1 <= depth_begin <= depth_end <= L, and depth_begin
 * must equal st->next_depth). At depth d every parent of depth d-1 (the root
 * for d = 1) scores all K candidates of position d:
 *   log q = log-softmax_K(cand_logit + <s_parent, U[cand]>),
 *   cum = cum_parent + log q,  s_beta = cum + beta*d,
 * the W best children under the comparator are kept (slot order), and for
 * d < L each survivor gets s = tanh(A s_parent + E[u] + h_d).
 * cand_ids/cand_logit as produced by dartree_topk_candidates (ids outside
 * [0, V) are read as 0); h[n][L][r] fp32 (row d is used by depth-d states, row
 * 0 is the root state). Writes levels depth_begin..depth_end of *st and, when
 * depth_end < L, st->state; advances st->next_depth to depth_end + 1. */
dartree_status dartree_expand_depth(const dartree_dims* dims, const dartree_head* head, const int32_t* cand_ids,
                                    const float* cand_logit, const float* h, dartree_supertree* st,
                                    int32_t depth_begin, int32_t depth_end, void* stream);

/* Steps a4 + a5 (marsggbo section 3.1, deferred pruning and Lemma 1): from the
 * complete supertree (all L depths expanded), select the min(B, nodes) best
 * nodes under the comparator (prefix-closed for beta <= 0) and emit them in
 * breadth-first order: depth ascending, then the parent's emitted index, then
 * token id. Outputs per request: n_sel[n]; tok, depth, parent, score, slot
 * [n][B] (parent -1 = the anchor token, slot = the node's slot in its supertree
 * level); entries >= n_sel are tok -1, depth 0, parent -2, score -inf,
 * slot -1. */
dartree_status dartree_select_topB(const dartree_dims* dims, const dartree_supertree* st, int32_t* n_sel,
                                   int32_t* tok, int32_t* depth, int32_t* parent, float* score, int32_t* slot,
                                   void* stream);

/* Step a5 (marsggbo section 3.2, tree-attention verification): ancestor
 * bitmask mask[n][B][ceil(B/64)] uint64. Row i (i < n_sel) has bit j (bit j%64
 * of word j/64) set iff j == i or node j is an ancestor of node i under the
 * parent array (the anchor, -1, has no bit); rows >= n_sel are zero. Parent
 * pointers outside [-1, i) end a chain. */
dartree_status dartree_tree_mask(const dartree_dims* dims, const int32_t* n_sel, const int32_t* parent,
                                 uint64_t* mask, void* stream);

/* The whole round (a0..a5) in one call. H_or_h is H[n][L][D] (weight_dtype)
 * when D > 0, else h[n][L][r] fp32. h receives the head inputs when D > 0
 * (may equal H_or_h's role otherwise and is then not written). Writes the
 * candidates, the supertree (st->next_depth must be 1; it ends at L + 1) and
 * the tree outputs of dartree_select_topB plus the mask. ws as for
 * dartree_topk_candidates. */
dartree_status dartree_build_round(const dartree_dims* dims, const dartree_head* head, const void* logits,
                                   const void* H_or_h, int32_t* cand_ids, float* cand_logit, float* h,
                                   dartree_supertree* st, int32_t* n_sel, int32_t* tok, int32_t* depth,
                                   int32_t* parent, float* score, int32_t* slot, uint64_t* mask, void* ws,
                                   size_t ws_bytes, void* stream);

/* dartree_build_round without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, meaning, layouts, outputs
 * and errors as dartree_build_round, minus ws / ws_bytes: the round's scratch
 * (the scan's sorted slice lists, the fp16 copy of A and, when it fits, the
 * split general kernel's exchange area) lives in a device array the library
 * owns, DARTREE_NOALLOC_SCRATCH_BYTES per GPU (each GPU the call runs on holds
 * its own copy until the process ends; the first call on a device looks its
 * address up). The call allocates and frees nothing. When the exchange area
 * does not fit, the general kernel keeps one workgroup a request (the same
 * results). Sizes whose scratch exceeds the array even without the exchange
 * area return DARTREE_ERR_UNSUPPORTED before anything is enqueued. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. The array keeps
 * the last call's contents; nothing in it has to start at zero. */
#define DARTREE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dartree_status dartree_build_round_noalloc(const dartree_dims* dims, const dartree_head* head, const void* logits,
                                           const void* H_or_h, int32_t* cand_ids, float* cand_logit, float* h,
                                           dartree_supertree* st, int32_t* n_sel, int32_t* tok, int32_t* depth,
                                           int32_t* parent, float* score, int32_t* slot, uint64_t* mask,
                                           void* stream);

/* How dartree_build_round runs for these sizes; a host-only query (no device
 * work, no allocation), valid whenever dartree_workspace_size succeeds.
 *   n_launches      kernel launches per round (2: scan, tree; 3 with a separate
 *                   merge of the scan's slice lists or a separate head projection)
 *   scan_slices     vocabulary slices per logits row (1 = one workgroup per row)
 *   scan_workgroups workgroups of the scan launch, head projection tiles and
 *                   (with the block-decoding tree kernel) the 16 that stage A
 *                   as fp16 MFMA fragments in the workspace included
 *   merge_separate  1 when the slice lists are merged by their own launch,
 *                   0 when the tree kernel merges them (or there is one slice)
 *   tree_kernel     1 = block-decoding kernel (K <= 64, W <= 16, r = 256, bf16
 *                   weights), 0 = general kernel
 *   tree_lds_bytes  dynamic LDS of the tree launch
 *   tree_parts      workgroups per request of the tree launch: the general
 *                   kernel with bf16 weights (r % 32 == 0) spreads a request
 *                   over up to 4 workgroups while n_req * parts <= 256, each
 *                   computing a share of the depth's contraction tiles and
 *                   exchanging them through the workspace; 1 otherwise
 * Errors: INVALID_ARGUMENT (bad dims or NULL info), UNSUPPORTED (no plan). */
typedef struct {
  int32_t n_launches, scan_slices, scan_workgroups, merge_separate, tree_kernel, tree_lds_bytes, tree_parts;
} dartree_round_info;
dartree_status dartree_round_plan(const dartree_dims* dims, dartree_round_info* info);

/* Heap-serial construction, the "pop then correct" baseline of the deferred
 * round (marsggbo blog, section 2 and section 4.3, Table 2: a best-first
 * builder that runs the correction head once per popped node). Per request,
 * from the round's candidates and head inputs: the root (state h_0) has the K
 * candidates of depth 1 as pending children; B times, the best pending node
 * by the round's comparator (s_beta descending, depth ascending, token
 * ascending, then the parent's own order) is popped; when its depth d < L its
 * state tanh(A s_parent + E[u] + h_d) is computed and all K candidates of
 * depth d + 1 become its pending children with
 * cum = cum_parent + min(log q, 0), s_beta = cum + beta (d + 1). No per-depth
 * width applies (W is ignored). With W >= B the deferred round selects the
 * same nodes (a consequence of the definitions, pinned on the oracle).
 * Inputs: cand_ids / cand_logit [n][L][K] (dartree_topk_candidates), h
 * [n][L][r] fp32 (dartree_head_states or supplied), the head (A, E, U in
 * weight_dtype). Outputs in pop order, device arrays [n][B]: tok, depth,
 * parent (pop index of the parent, -1 for the root; always below the node's
 * own index), score (s_beta); n_sel[n] = min(B, reachable nodes); pads as in
 * dartree_select_topB (tok -1, depth 0, parent -2, score -inf).
 * dartree_tree_mask builds the ancestor mask from n_sel and parent. ws is a
 * device workspace of dartree_serial_workspace_size bytes (the nodes' states,
 * [n][B + 1][r] fp32), overwritten. UNSUPPORTED for B > 511; other errors as
 * for the round. */
dartree_status dartree_serial_workspace_size(const dartree_dims* dims, size_t* bytes);
dartree_status dartree_build_serial(const dartree_dims* dims, const dartree_head* head, const int32_t* cand_ids,
                                    const float* cand_logit, const float* h, int32_t* n_sel, int32_t* tok,
                                    int32_t* depth, int32_t* parent, float* score, void* ws, size_t ws_bytes,
                                    void* stream);

/* Verification consumer of an emitted tree with a synthetic target
 * (marsggbo blog, section 3.2: the target verifies the drafted tree in one
 * pass under the tree-attention mask and keeps the longest root path it
 * agrees with). Per request:
 *   acceptance  target[n][L] int32 is the target's continuation (its token at
 *               depth d is target[d-1]); a node is accepted iff its token equals
 *               the target's at its depth and its parent is the anchor (-1) or
 *               accepted. accepted_len[n] = 1 + the depth of the deepest
 *               accepted node (the target's own next token counts);
 *               accepted_nodes[n][L] = the emitted indices along that path,
 *               depth 1 first, -1 past its end.
 *   attention   one head over the draft nodes: attn_out[i] = sum_j
 *               softmax_j(<Q[i], K[j]> / sqrt(dh)) V[j] over the j whose bit
 *               is set in mask row i (dartree_tree_mask layout: the node and its
 *               ancestors); rows >= n_sel are zero. Q, K, V, attn_out are
 *               [n][B][dh] fp32, 1 <= dh <= 256 (UNSUPPORTED otherwise).
 * The tree (n_sel, tok, depth, parent, mask) is an emitted round
 * (dartree_build_round, or dartree_select_topB + dartree_tree_mask); parent
 * indices below their node's, as emitted. Device pointers, caller-owned. */
dartree_status dartree_verify_tree(const dartree_dims* dims, const int32_t* n_sel, const int32_t* tok,
                                   const int32_t* depth, const int32_t* parent, const uint64_t* mask,
                                   const int32_t* target, const float* Q, const float* K, const float* V, int32_t dh,
                                   int32_t* accepted_len, int32_t* accepted_nodes, float* attn_out, void* stream);

/* Measurement utility (not part of a round's computation): one read-only
 * pass over `bytes` bytes (a positive multiple of 16) at the device pointer
 * buf (16-byte aligned), 16-byte vector loads, 256 workgroups of 512 threads;
 * the achievable HBM read rate the logits scan and the LM head are compared
 * with. sink is a device word the kernel may write (never in practice). */
dartree_status dartree_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Measurement utility (not part of a round's computation): the same read as
 * dartree_stream_read by a single workgroup of 1024 threads, eight 16-byte
 * loads in flight a thread: the rate one CU pulls from the memory system,
 * which bounds the block-decoding tree kernel (one workgroup a request).
 * Same arguments and errors as dartree_stream_read. */
dartree_status dartree_cu_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Profiling hook (not part of a round's computation). When set, every
 * following dartree_build_round on this thread records events[0] before its
 * first launch, events[1] after the logits scan (with the head tiles),
 * events[2] after the candidate merge (recorded also when no merge runs) and
 * events[3] after the tree kernel, each on the call's stream, so that
 * hipEventElapsedTime gives the time of each stage; every following
 * dartree_topk_candidates records events[0], events[1] (after the scan) and
 * events[2] (after the merge) the same way. `events` holds n = 4
 * hipEvent_t handles (passed as void*) created by the caller and kept alive
 * while set; n = 0 (events may be NULL) clears the hook. Returns
 * INVALID_ARGUMENT for any other n or NULL handles. */
dartree_status dartree_set_stage_events(void* const* events, int32_t n);

/* Bound, in microseconds (0 .. 1000000, default 200), of how long a
 * workgroup of the split general tree kernel (dartree_round_info.tree_parts
 * > 1) waits for another part of its request to publish a depth's
 * contraction slice before computing that slice itself; a part that missed
 * the bound is not waited for again in that launch. Results do not depend on
 * it: 0 makes every part compute the whole contraction (the path a part takes
 * when its partners are not resident, e.g. on a GPU shared with other work).
 * Process-wide; applies to rounds launched after the call. INVALID_ARGUMENT
 * outside the range. */
dartree_status dartree_set_split_wait(int32_t microseconds);

#ifdef __cplusplus
}
#endif

#endif /* DARTREE_H */
