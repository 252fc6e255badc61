// C ABI of libdartree: argument validation, workspace layout and kernel
// dispatch. Every entry point validates completely before it enqueues.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/dartree.h"
#include "kernels.h"

namespace dartree {
// measurement utility (lmhead.hip, beside the HBM read probe): one read of
// bytes (a multiple of 16) at buf by a single workgroup
hipError_t launch_cu_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
}  // namespace dartree

#include "api_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_stage_ev[4] = {nullptr, nullptr, nullptr, nullptr};
thread_local bool g_stage_on = false;
// bound of the split tree kernel's wait for another part's slice (microseconds)
std::atomic<uint32_t> g_split_wait_us{200};

void stage_mark(int i, hipStream_t s) {
  if (g_stage_on) (void)hipEventRecord(g_stage_ev[i], s);
}

dartree_status fail(dartree_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dartree_status hip_fail(hipError_t e, const char* what) {
  return fail(DARTREE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQ_PTR(p, a)                                                                          \
  do {                                                                                         \
    if ((p) == nullptr) return fail(DARTREE_ERR_INVALID_ARGUMENT, "%s is NULL", #p);           \
    if (!aligned((p), (a)))                                                                    \
      return fail(DARTREE_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #p, (int)(a));    \
  } while (0)

constexpr int kMaxL = 31, kMaxK = 1024, kMaxW = 64, kMaxB = 1024, kMaxR = 1024, kMaxV = 1 << 18;

dartree_status check_dims(const dartree_dims* d) {
  if (!d) return fail(DARTREE_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->n_req < 1 || d->L < 1 || d->V < 1 || d->K < 1 || d->W < 1 || d->B < 1 || d->r < 1 || d->D < 0)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "sizes must be positive (n_req=%d L=%d V=%d K=%d W=%d B=%d r=%d D=%d)",
                d->n_req, d->L, d->V, d->K, d->W, d->B, d->r, d->D);
  if (d->K > d->V) return fail(DARTREE_ERR_INVALID_ARGUMENT, "K=%d exceeds V=%d", d->K, d->V);
  if (!std::isfinite(d->beta)) return fail(DARTREE_ERR_INVALID_ARGUMENT, "beta is not finite");
  if (d->beta > 0.f)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "beta=%g > 0: prefix closure (Lemma 1) needs beta <= 0", d->beta);
  if ((d->logits_dtype != DARTREE_F32 && d->logits_dtype != DARTREE_BF16) ||
      (d->weight_dtype != DARTREE_F32 && d->weight_dtype != DARTREE_BF16))
    return fail(DARTREE_ERR_UNSUPPORTED, "unknown dtype");
  if (d->L > kMaxL || d->K > kMaxK || d->W > kMaxW || d->B > kMaxB || d->r > kMaxR || d->V > kMaxV ||
      d->n_req > 65535 || d->D > (1 << 20))
    return fail(DARTREE_ERR_UNSUPPORTED,
                "limits: L<=%d K<=%d W<=%d B<=%d r<=%d V<=%d n_req<=65535 D<=2^20 (got L=%d K=%d W=%d B=%d r=%d V=%d)",
                kMaxL, kMaxK, kMaxW, kMaxB, kMaxR, kMaxV, d->L, d->K, d->W, d->B, d->r, d->V);
  if (d->W * d->r > 8192 || d->W * d->K > 8192)
    return fail(DARTREE_ERR_UNSUPPORTED, "limits: W*r <= 8192 and W*K <= 8192 (got W*r=%d W*K=%d)", d->W * d->r,
                d->W * d->K);
  return DARTREE_OK;
}

struct WsLayout {
  dartree::ScanPlan plan;
  size_t lists_off, afrag_off, total;   // afrag_off = 0: no A fragment copy
  int split;                            // general kernel: workgroups per request
  size_t xch_off, xflag_off;            // its exchange slices and flags (split > 1)
};

// The general MFMA tree kernel (bf16 weights, r % 32 == 0, outside the
// block-decoding shapes) spreads a request over up to 4 workgroups while
// n_req * parts stays within the 256 compute units of an MI355X.
int split_parts(const dartree_dims* d) {
  if (d->weight_dtype != DARTREE_BF16 || d->r % 32 != 0) return 1;
  if (d->r == 256 && (d->K == 16 || d->K == 32 || d->K == 64) && d->W <= 16) return 1;
  const int per = 256 / d->n_req;
  return per >= 4 ? 4 : per >= 2 ? 2 : 1;
}

WsLayout ws_layout(const dartree_dims* d, bool allow_split = true) {
  WsLayout w{};
  const int rows = d->n_req * d->L;
  w.plan = dartree::scan_plan(rows, d->V, d->K, d->logits_dtype == DARTREE_BF16);
  w.lists_off = 0;
  w.total = (w.plan.list_bytes + 255) & ~(size_t)255;
  // bf16 weights of rank 256: room for the fp16 A fragments the scan launch
  // stages for the block-decoding tree kernel
  if (d->weight_dtype == DARTREE_BF16 && d->r == 256) {
    if (w.total == 0) w.total = 256;
    w.afrag_off = w.total;
    w.total += dartree::kAFragBytes;
  }
  if (w.total == 0) w.total = 256;
  w.split = allow_split ? split_parts(d) : 1;
  if (w.split > 1) {
    w.xch_off = w.total;
    const size_t row = (size_t)(d->K + 15) / 16 * 16 + d->r;   // Z blocks, then AS
    w.total += ((size_t)d->n_req * d->L * d->W * row * sizeof(float) + 255) & ~(size_t)255;
    w.xflag_off = w.total;
    w.total += ((size_t)d->n_req * w.split * d->L * sizeof(uint32_t) + 255) & ~(size_t)255;
  }
  return w;
}

dartree_status check_ws(const dartree_dims* d, void* ws, size_t ws_bytes, WsLayout* out, bool allow_split = true) {
  *out = ws_layout(d, allow_split);
  if (!out->plan.ok) return fail(DARTREE_ERR_UNSUPPORTED, "no top-K plan for V=%d K=%d", d->V, d->K);
  REQ_PTR(ws, 256);
  if (ws_bytes < out->total)
    return fail(DARTREE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes, out->total);
  return DARTREE_OK;
}

dartree_status check_head(const dartree_dims* d, const dartree_head* h) {
  if (!h) return fail(DARTREE_ERR_INVALID_ARGUMENT, "head is NULL");
  if (h->flags & ~DARTREE_HEAD_EXACT) return fail(DARTREE_ERR_INVALID_ARGUMENT, "unknown head flags 0x%x", h->flags);
  if (h->A != nullptr) REQ_PTR(h->A, 16);   // NULL: the Markov head (A = 0)
  REQ_PTR(h->E, 16);
  REQ_PTR(h->U, 16);
  (void)d;
  return DARTREE_OK;
}

dartree_status check_supertree(const dartree_supertree* st) {
  if (!st) return fail(DARTREE_ERR_INVALID_ARGUMENT, "supertree is NULL");
  REQ_PTR(st->tok, 4);
  REQ_PTR(st->parent_slot, 4);
  REQ_PTR(st->cum, 4);
  REQ_PTR(st->sbeta, 4);
  REQ_PTR(st->count, 4);
  REQ_PTR(st->state, 16);
  return DARTREE_OK;
}

dartree_status check_tree_out(const int32_t* n_sel, const int32_t* tok, const int32_t* depth, const int32_t* parent,
                              const float* score, const int32_t* slot) {
  REQ_PTR(n_sel, 4);
  REQ_PTR(tok, 4);
  REQ_PTR(depth, 4);
  REQ_PTR(parent, 4);
  REQ_PTR(score, 4);
  REQ_PTR(slot, 4);
  return DARTREE_OK;
}

#define TRY(x)                                \
  do {                                        \
    dartree_status _s = (x);                  \
    if (_s != DARTREE_OK) return _s;          \
  } while (0)

dartree::TreeArgs tree_args(const dartree_dims* dims, const dartree_head* head, const int32_t* cand_ids,
                           const float* cand_logit, const float* h, const dartree_supertree* st, int d0, int d1) {
  dartree::TreeArgs a{};
  a.n_req = dims->n_req;
  a.L = dims->L;
  a.V = dims->V;
  a.K = dims->K;
  a.W = dims->W;
  a.B = dims->B;
  a.r = dims->r;
  a.beta = dims->beta;
  a.bf16 = dims->weight_dtype == DARTREE_BF16;
  if (head) {
    a.exact = (head->flags & DARTREE_HEAD_EXACT) != 0;
    a.A = head->A;
    a.E = head->E;
    a.U = head->U;
  }
  a.cand_ids = cand_ids;
  a.cand_logit = cand_logit;
  a.h = h;
  a.st_tok = st->tok;
  a.st_parent = st->parent_slot;
  a.st_cum = st->cum;
  a.st_sbeta = st->sbeta;
  a.st_count = st->count;
  a.st_state = st->state;
  a.w_req = st->width;
  a.b_req = st->budget;
  a.d0 = d0;
  a.d1 = d1;
  a.split = 1;
  return a;
}

void set_tree_out(dartree::TreeArgs& a, int32_t* n_sel, int32_t* tok, int32_t* depth, int32_t* parent, float* score,
                  int32_t* slot, uint64_t* mask) {
  a.do_select = true;
  a.do_mask = mask != nullptr;
  a.n_sel = n_sel;
  a.tok = tok;
  a.depth = depth;
  a.parent = parent;
  a.score = score;
  a.slot = slot;
  a.mask = mask;
}

dartree_status check_tree_plan(const dartree::TreeArgs& a, dartree::TreePlan* p) {
  *p = dartree::tree_plan(a);
  if (!p->ok)
    return fail(DARTREE_ERR_UNSUPPORTED, "working set of %zu bytes exceeds the 160 KiB of LDS (K=%d W=%d r=%d L=%d B=%d)",
                p->smem, a.K, a.W, a.r, a.L, a.B);
  return DARTREE_OK;
}

// The launches of a round: the scan, then either the block-decoding tree
// kernel merging the scan's slice lists in its prologue, or (other plans) a
// separate merge launch ahead of the tree kernel.
dartree_status plan_round(const WsLayout& w, bool lbf, uint64_t* lists, int32_t* cand_ids, float* cand_logit,
                          dartree::TreeArgs& ta, dartree::TreePlan* tp) {
  if (w.plan.S > 1) {
    ta.lists = lists;
    ta.S = w.plan.S;
    ta.lbf16 = lbf;
    ta.cand_ids_out = cand_ids;
    ta.cand_logit_out = cand_logit;
  }
  *tp = dartree::tree_plan(ta);
  if (!(tp->ok && tp->mode == 3)) {
    // the lists go to their own merge launch; plan the tree kernel without them
    ta.lists = nullptr;
    ta.S = 0;
    *tp = dartree::tree_plan(ta);
  }
  return check_tree_plan(ta, tp);
}

}  // namespace

extern "C" {

const char* dartree_status_string(dartree_status s) {
  switch (s) {
    case DARTREE_OK: return "DARTREE_OK";
    case DARTREE_ERR_INVALID_ARGUMENT: return "DARTREE_ERR_INVALID_ARGUMENT";
    case DARTREE_ERR_UNSUPPORTED: return "DARTREE_ERR_UNSUPPORTED";
    case DARTREE_ERR_WORKSPACE_TOO_SMALL: return "DARTREE_ERR_WORKSPACE_TOO_SMALL";
    case DARTREE_ERR_HIP: return "DARTREE_ERR_HIP";
  }
  return "DARTREE_UNKNOWN_STATUS";
}

const char* dartree_last_error(void) { return g_err; }

int32_t dartree_version(void) { return 4; }

dartree_status dartree_round_plan(const dartree_dims* dims, dartree_round_info* info) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  if (!info) return fail(DARTREE_ERR_INVALID_ARGUMENT, "info is NULL");
  WsLayout w = ws_layout(dims);
  if (!w.plan.ok) return fail(DARTREE_ERR_UNSUPPORTED, "no top-K plan for V=%d K=%d", dims->V, dims->K);
  dartree_supertree st{};
  dartree::TreeArgs ta = tree_args(dims, nullptr, nullptr, nullptr, nullptr, &st, 1, dims->L);
  set_tree_out(ta, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, reinterpret_cast<uint64_t*>(256));
  if (w.split > 1) {
    ta.split = w.split;
    ta.xch = reinterpret_cast<float*>(256);
    ta.xflag = reinterpret_cast<uint32_t*>(256);
  }
  dartree::TreePlan tp;
  alignas(16) static uint64_t dummy_lists[2];
  TRY(plan_round(w, dims->logits_dtype == DARTREE_BF16, dummy_lists, nullptr, nullptr, ta, &tp));
  const bool merge_sep = w.plan.S > 1 && ta.lists == nullptr;
  info->scan_slices = w.plan.S;
  info->merge_separate = merge_sep ? 1 : 0;
  const int rows = dims->n_req * dims->L;
  const bool head_fused = dims->D > 0 && dartree::head_mfma_ok(dims->weight_dtype == DARTREE_BF16,
                                                               dummy_lists, dummy_lists, dims->D, dims->r);
  info->n_launches = 2 + (merge_sep ? 1 : 0) + ((dims->D > 0 && !head_fused) ? 1 : 0);
  const bool head_big = w.plan.wide && dartree::head_big_ok(rows, dims->D, dims->r);
  info->scan_workgroups = w.plan.n_scan + (head_fused ? dartree::head_tiles(head_big, rows, dims->r) : 0) +
                          ((tp.mode == 3 && w.afrag_off) ? dartree::kAFragWaves : 0);
  info->tree_kernel = tp.mode == 3 ? 1 : 0;
  info->tree_lds_bytes = (int32_t)tp.smem;
  info->tree_parts = tp.mode == 1 ? tp.split : 1;
  return DARTREE_OK;
}

dartree_status dartree_set_stage_events(void* const* events, int32_t n) {
  g_err[0] = 0;
  if (n == 0) {
    g_stage_on = false;
    return DARTREE_OK;
  }
  if (n != 4 || !events) return fail(DARTREE_ERR_INVALID_ARGUMENT, "stage events: need n = 4 handles (or n = 0)");
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return fail(DARTREE_ERR_INVALID_ARGUMENT, "stage event %d is NULL", i);
  for (int i = 0; i < 4; ++i) g_stage_ev[i] = static_cast<hipEvent_t>(events[i]);
  g_stage_on = true;
  return DARTREE_OK;
}

dartree_status dartree_set_split_wait(int32_t microseconds) {
  g_err[0] = 0;
  if (microseconds < 0 || microseconds > 1000000)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "split wait of %d us: 0 .. 1000000", microseconds);
  g_split_wait_us.store((uint32_t)microseconds);
  return DARTREE_OK;
}

dartree_status dartree_workspace_size(const dartree_dims* dims, size_t* bytes) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  if (!bytes) return fail(DARTREE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  WsLayout w = ws_layout(dims);
  if (!w.plan.ok) return fail(DARTREE_ERR_UNSUPPORTED, "no top-K plan for V=%d K=%d", dims->V, dims->K);
  *bytes = w.total;
  return DARTREE_OK;
}

dartree_status dartree_workspace_init(const dartree_dims* dims, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  WsLayout w;
  TRY(check_ws(dims, ws, ws_bytes, &w));
  (void)stream;   // the current kernels keep no state in the workspace between calls
  return DARTREE_OK;
}

dartree_status dartree_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  g_err[0] = 0;
  REQ_PTR(buf, 16);
  REQ_PTR(sink, 4);
  if (bytes == 0 || bytes % 16 != 0) return fail(DARTREE_ERR_INVALID_ARGUMENT, "bytes=%zu: a positive multiple of 16", bytes);
  hipError_t e = dartree::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return DARTREE_OK;
}

dartree_status dartree_cu_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  g_err[0] = 0;
  REQ_PTR(buf, 16);
  REQ_PTR(sink, 4);
  if (bytes == 0 || bytes % 16 != 0) return fail(DARTREE_ERR_INVALID_ARGUMENT, "bytes=%zu: a positive multiple of 16", bytes);
  hipError_t e = dartree::launch_cu_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cu read launch");
  return DARTREE_OK;
}

dartree_status dartree_head_check(const dartree_dims* dims, const dartree_head* head, int32_t* flags, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  TRY(check_head(dims, head));
  REQ_PTR(flags, 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dims->weight_dtype == DARTREE_BF16
                     ? dartree::launch_head_check(static_cast<const uint16_t*>(head->A),
                                                  static_cast<const uint16_t*>(head->U), dims->V, dims->r, flags, s)
                     : dartree::launch_fill_u32(flags, 1, 0u, s);
  if (e != hipSuccess) return hip_fail(e, "head check launch");
  return DARTREE_OK;
}

dartree_status dartree_head_states(const dartree_dims* dims, const void* H, const void* Pt, float* h, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  if (dims->D < 1) return fail(DARTREE_ERR_INVALID_ARGUMENT, "head_states needs D >= 1");
  REQ_PTR(H, 16);
  REQ_PTR(Pt, 16);
  REQ_PTR(h, 4);
  hipError_t e = dartree::launch_head(dims->weight_dtype == DARTREE_BF16, H, Pt, h, dims->n_req * dims->L, dims->D,
                                      dims->r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "head_states launch");
  return DARTREE_OK;
}

dartree_status dartree_topk_candidates(const dartree_dims* dims, const void* logits, int32_t* cand_ids,
                                       float* cand_logit, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  REQ_PTR(logits, 16);
  REQ_PTR(cand_ids, 4);
  REQ_PTR(cand_logit, 4);
  WsLayout w;
  TRY(check_ws(dims, ws, ws_bytes, &w));
  const bool bf = dims->logits_dtype == DARTREE_BF16;
  const int rows = dims->n_req * dims->L;
  dartree::ScanArgs sa{};
  sa.logits = logits;
  sa.rows = rows;
  sa.V = dims->V;
  sa.K = dims->K;
  sa.lists = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + w.lists_off);
  sa.cand_ids = cand_ids;
  sa.cand_logit = cand_logit;
  hipStream_t s = static_cast<hipStream_t>(stream);
  stage_mark(0, s);
  hipError_t e = dartree::launch_scan(w.plan, bf, sa, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  stage_mark(1, s);
  e = dartree::launch_merge(w.plan, rows, dims->K, bf, sa.lists, cand_ids, cand_logit, s);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  stage_mark(2, s);
  return DARTREE_OK;
}

dartree_status lmhead_check(const dartree_dims* dims, dartree::LmheadPlan* p) {
  TRY(check_dims(dims));
  if (dims->weight_dtype != DARTREE_BF16)
    return fail(DARTREE_ERR_UNSUPPORTED, "the fused LM head takes bf16 hidden states and head rows");
  *p = dartree::lmhead_plan(dims->n_req * dims->L, dims->V, dims->D, dims->K);
  if (!p->ok)
    return fail(DARTREE_ERR_UNSUPPORTED,
                "fused LM head limits: K <= 64, D >= 256 and a multiple of 256, V <= 262144 (got K=%d D=%d V=%d)",
                dims->K, dims->D, dims->V);
  return DARTREE_OK;
}

dartree_status dartree_lmhead_workspace_size(const dartree_dims* dims, size_t* bytes) {
  g_err[0] = 0;
  dartree::LmheadPlan p;
  TRY(lmhead_check(dims, &p));
  if (!bytes) return fail(DARTREE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = (p.list_bytes + 255) & ~(size_t)255;
  return DARTREE_OK;
}

dartree_status dartree_lmhead_topk(const dartree_dims* dims, const void* X, const void* Wlm, int32_t* cand_ids,
                                   float* cand_logit, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  dartree::LmheadPlan p;
  TRY(lmhead_check(dims, &p));
  REQ_PTR(X, 16);
  REQ_PTR(Wlm, 16);
  REQ_PTR(cand_ids, 4);
  REQ_PTR(cand_logit, 4);
  REQ_PTR(ws, 256);
  if (ws_bytes < p.list_bytes)
    return fail(DARTREE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes, p.list_bytes);
  hipError_t e = dartree::launch_lmhead_topk(p, static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wlm),
                                             dims->n_req * dims->L, dims->V, dims->D, dims->K,
                                             static_cast<uint64_t*>(ws), cand_ids, cand_logit,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "lmhead launch");
  return DARTREE_OK;
}

dartree_status dartree_expand_depth(const dartree_dims* dims, const dartree_head* head, const int32_t* cand_ids,
                                    const float* cand_logit, const float* h, dartree_supertree* st,
                                    int32_t depth_begin, int32_t depth_end, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  TRY(check_head(dims, head));
  REQ_PTR(cand_ids, 4);
  REQ_PTR(cand_logit, 4);
  REQ_PTR(h, 16);
  TRY(check_supertree(st));
  if (depth_begin != st->next_depth)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "depth_begin=%d but the supertree expects depth %d", depth_begin,
                st->next_depth);
  if (depth_begin < 1 || depth_end < depth_begin || depth_end > dims->L)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "depth range [%d, %d] outside [1, %d]", depth_begin, depth_end, dims->L);
  dartree::TreeArgs ta = tree_args(dims, head, cand_ids, cand_logit, h, st, depth_begin, depth_end);
  dartree::TreePlan tp;
  TRY(check_tree_plan(ta, &tp));
  hipError_t e = dartree::launch_tree(tp, ta, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "expand launch");
  st->next_depth = depth_end + 1;
  return DARTREE_OK;
}

dartree_status dartree_select_topB(const dartree_dims* dims, const dartree_supertree* st, int32_t* n_sel,
                                   int32_t* tok, int32_t* depth, int32_t* parent, float* score, int32_t* slot,
                                   void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  TRY(check_supertree(st));
  if (st->next_depth != dims->L + 1)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "supertree incomplete: next_depth=%d, expected %d", st->next_depth,
                dims->L + 1);
  TRY(check_tree_out(n_sel, tok, depth, parent, score, slot));
  dartree::TreeArgs ta = tree_args(dims, nullptr, nullptr, nullptr, nullptr, st, 1, 0);
  set_tree_out(ta, n_sel, tok, depth, parent, score, slot, nullptr);
  dartree::TreePlan tp;
  TRY(check_tree_plan(ta, &tp));
  hipError_t e = dartree::launch_tree(tp, ta, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return DARTREE_OK;
}

dartree_status dartree_tree_mask(const dartree_dims* dims, const int32_t* n_sel, const int32_t* parent,
                                 uint64_t* mask, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  REQ_PTR(n_sel, 4);
  REQ_PTR(parent, 4);
  REQ_PTR(mask, 8);
  hipError_t e = dartree::launch_mask(dims->n_req, dims->B, n_sel, parent, mask, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask launch");
  return DARTREE_OK;
}

dartree_status dartree_build_round(const dartree_dims* dims, const dartree_head* head, const void* logits,
                                   const void* H_or_h, int32_t* cand_ids, float* cand_logit, float* h,
                                   dartree_supertree* st, int32_t* n_sel, int32_t* tok, int32_t* depth,
                                   int32_t* parent, float* score, int32_t* slot, uint64_t* mask, void* ws,
                                   size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return dartree::build_round_impl(dims, head, logits, H_or_h, cand_ids, cand_logit, h, st, n_sel, tok, depth,
                                   parent, score, slot, mask, ws, ws_bytes, stream);
}

}  // extern "C"

namespace dartree {

dartree_status set_error(dartree_status s, const char* msg) { return fail(s, "%s", msg); }

size_t round_workspace_bytes(const dartree_dims* dims, bool allow_split) {
  return ws_layout(dims, allow_split).total;
}

dartree_status check_round_dims(const dartree_dims* dims) {
  TRY(check_dims(dims));
  if (!ws_layout(dims).plan.ok) return fail(DARTREE_ERR_UNSUPPORTED, "no top-K plan for V=%d K=%d", dims->V, dims->K);
  return DARTREE_OK;
}

dartree_status build_round_impl(const dartree_dims* dims, const dartree_head* head, const void* logits,
                                const void* H_or_h, int32_t* cand_ids, float* cand_logit, float* h,
                                dartree_supertree* st, int32_t* n_sel, int32_t* tok, int32_t* depth,
                                int32_t* parent, float* score, int32_t* slot, uint64_t* mask, void* ws,
                                size_t ws_bytes, void* stream, bool allow_split) {
  TRY(check_dims(dims));
  TRY(check_head(dims, head));
  REQ_PTR(logits, 16);
  REQ_PTR(H_or_h, 16);
  REQ_PTR(cand_ids, 4);
  REQ_PTR(cand_logit, 4);
  if (dims->D > 0) {
    REQ_PTR(h, 16);
    REQ_PTR(head->Pt, 16);
  }
  TRY(check_supertree(st));
  if (st->next_depth != 1)
    return fail(DARTREE_ERR_INVALID_ARGUMENT, "supertree next_depth=%d, a round starts at 1", st->next_depth);
  TRY(check_tree_out(n_sel, tok, depth, parent, score, slot));
  REQ_PTR(mask, 8);
  WsLayout w;
  TRY(check_ws(dims, ws, ws_bytes, &w, allow_split));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool lbf = dims->logits_dtype == DARTREE_BF16, wbf = dims->weight_dtype == DARTREE_BF16;
  const int rows = dims->n_req * dims->L;
  const float* hin = static_cast<const float*>(H_or_h);
  dartree::TreeArgs ta = tree_args(dims, head, cand_ids, cand_logit, dims->D > 0 ? h : hin, st, 1, dims->L);
  set_tree_out(ta, n_sel, tok, depth, parent, score, slot, mask);
  if (w.split > 1) {
    ta.split = w.split;
    ta.xch = reinterpret_cast<float*>(static_cast<char*>(ws) + w.xch_off);
    ta.xflag = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + w.xflag_off);
    ta.split_wait = g_split_wait_us.load() * 100u;
  }
  uint64_t* lists = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + w.lists_off);
  dartree::TreePlan tp;
  TRY(plan_round(w, lbf, lists, cand_ids, cand_logit, ta, &tp));
  uint16_t* a_frag = (tp.mode == 3 && w.afrag_off && head->A != nullptr)
                         ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + w.afrag_off)
                         : nullptr;
  ta.a_frag = a_frag;
  // launch 1: the logits scan, with the head projection tiles riding along
  dartree::ScanArgs sa{};
  sa.logits = logits;
  sa.rows = rows;
  sa.V = dims->V;
  sa.K = dims->K;
  sa.lists = lists;
  if (a_frag) {
    sa.A = static_cast<const uint16_t*>(head->A);
    sa.a_frag = a_frag;
    sa.n_afrag = dartree::kAFragWaves;
  }
  sa.cand_ids = cand_ids;
  sa.cand_logit = cand_logit;
  if (tp.mode == 1 && tp.split > 1) {
    // the split tree kernel's flags start at zero
    sa.clear = ta.xflag;
    sa.n_clear = dims->n_req * tp.split * dims->L;
  }
  const bool fuse_head = dims->D > 0 && dartree::head_mfma_ok(wbf, H_or_h, head->Pt, dims->D, dims->r);
  if (fuse_head) {
    sa.H = static_cast<const uint16_t*>(H_or_h);
    sa.Pt = static_cast<const uint16_t*>(head->Pt);
    sa.h = h;
    sa.M = rows;
    sa.D = dims->D;
    sa.r = dims->r;
    sa.head_big = (w.plan.wide && dartree::head_big_ok(rows, dims->D, dims->r)) ? 1 : 0;
    sa.n_head = dartree::head_tiles(sa.head_big, rows, dims->r);
  }
  hipError_t e;
  stage_mark(0, s);
  if (dims->D > 0 && !fuse_head) {
    e = dartree::launch_head_valu(wbf, H_or_h, head->Pt, h, rows, dims->D, dims->r, s);
    if (e != hipSuccess) return hip_fail(e, "head launch");
  }
  e = dartree::launch_scan(w.plan, lbf, sa, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  stage_mark(1, s);
  if (!ta.lists) {
    e = dartree::launch_merge(w.plan, rows, dims->K, lbf, sa.lists, cand_ids, cand_logit, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  stage_mark(2, s);
  // launch 2: expansion, selection, emission and mask, one workgroup per request
  e = dartree::launch_tree(tp, ta, s);
  if (e != hipSuccess) return hip_fail(e, "tree launch");
  stage_mark(3, s);
  st->next_depth = dims->L + 1;
  return DARTREE_OK;
}

}  // namespace dartree

extern "C" {

dartree_status dartree_serial_workspace_size(const dartree_dims* dims, size_t* bytes) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  if (!bytes) return fail(DARTREE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = (size_t)dims->n_req * (size_t)(dims->B + 1) * (size_t)dims->r * sizeof(float);
  return DARTREE_OK;
}

dartree_status dartree_build_serial(const dartree_dims* dims, const dartree_head* head, const int32_t* cand_ids,
                                    const float* cand_logit, const float* h, int32_t* n_sel, int32_t* tok,
                                    int32_t* depth, int32_t* parent, float* score, void* ws, size_t ws_bytes,
                                    void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  if (dims->B > dartree::kSerialMaxB)
    return fail(DARTREE_ERR_UNSUPPORTED, "heap-serial construction: B=%d exceeds %d", dims->B, dartree::kSerialMaxB);
  if (!head) return fail(DARTREE_ERR_INVALID_ARGUMENT, "head is NULL");
  const int wa = dims->weight_dtype == DARTREE_BF16 ? 2 : 4;
  if (head->A != nullptr) REQ_PTR(head->A, wa);   // NULL: the Markov head (A = 0)
  REQ_PTR(head->E, wa);
  REQ_PTR(head->U, wa);
  REQ_PTR(cand_ids, 4);
  REQ_PTR(cand_logit, 4);
  REQ_PTR(h, 4);
  REQ_PTR(n_sel, 4);
  REQ_PTR(tok, 4);
  REQ_PTR(depth, 4);
  REQ_PTR(parent, 4);
  REQ_PTR(score, 4);
  REQ_PTR(ws, 4);
  const size_t need = (size_t)dims->n_req * (size_t)(dims->B + 1) * (size_t)dims->r * sizeof(float);
  if (ws_bytes < need)
    return fail(DARTREE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  dartree::SerialArgs a{};
  a.n_req = dims->n_req;
  a.L = dims->L;
  a.V = dims->V;
  a.K = dims->K;
  a.B = dims->B;
  a.r = dims->r;
  a.beta = dims->beta;
  a.A = head->A;
  a.E = head->E;
  a.U = head->U;
  a.cand_ids = cand_ids;
  a.cand_logit = cand_logit;
  a.h = h;
  a.states = static_cast<float*>(ws);
  a.n_sel = n_sel;
  a.tok = tok;
  a.depth = depth;
  a.parent = parent;
  a.score = score;
  hipError_t e = dartree::launch_serial(a, dims->weight_dtype == DARTREE_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "serial launch");
  return DARTREE_OK;
}

dartree_status dartree_verify_tree(const dartree_dims* dims, const int32_t* n_sel, const int32_t* tok,
                                   const int32_t* depth, const int32_t* parent, const uint64_t* mask,
                                   const int32_t* target, const float* Q, const float* K, const float* V, int32_t dh,
                                   int32_t* accepted_len, int32_t* accepted_nodes, float* attn_out, void* stream) {
  g_err[0] = 0;
  TRY(check_dims(dims));
  if (dh < 1 || dh > 256) return fail(DARTREE_ERR_UNSUPPORTED, "dh=%d outside 1..256", dh);
  REQ_PTR(n_sel, 4);
  REQ_PTR(tok, 4);
  REQ_PTR(depth, 4);
  REQ_PTR(parent, 4);
  REQ_PTR(mask, 8);
  REQ_PTR(target, 4);
  REQ_PTR(Q, 4);
  REQ_PTR(K, 4);
  REQ_PTR(V, 4);
  REQ_PTR(accepted_len, 4);
  REQ_PTR(accepted_nodes, 4);
  REQ_PTR(attn_out, 4);
  dartree::VerifyArgs a{};
  a.n_req = dims->n_req;
  a.L = dims->L;
  a.B = dims->B;
  a.dh = dh;
  a.n_sel = n_sel;
  a.tok = tok;
  a.depth = depth;
  a.parent = parent;
  a.mask = mask;
  a.target = target;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.acc_len = accepted_len;
  a.acc_nodes = accepted_nodes;
  a.out = attn_out;
  hipError_t e = dartree::launch_verify(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "verify launch");
  return DARTREE_OK;
}

}  // extern "C"
