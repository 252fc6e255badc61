// Entry-point helpers shared between the C ABI's translation units (internal
// to libdartree).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/dartree.h"

namespace dartree {

// The whole round behind dartree_build_round: full validation, then the
// launches, with `ws` (ws_bytes) as the round's scratch. allow_split = false
// keeps the general tree kernel at one workgroup per request (no exchange
// area in the scratch).
dartree_status build_round_impl(const dartree_dims* dims, const dartree_head* head, const void* logits,
                                const void* H_or_h, int32_t* cand_ids, float* cand_logit, float* h,
                                dartree_supertree* st, int32_t* n_sel, int32_t* tok, int32_t* depth,
                                int32_t* parent, float* score, int32_t* slot, uint64_t* mask, void* ws,
                                size_t ws_bytes, void* stream, bool allow_split = true);
// dims valid and a top-K plan exists (else the status, with the detail set)
dartree_status check_round_dims(const dartree_dims* dims);
// scratch bytes a round of these (valid) dims needs
size_t round_workspace_bytes(const dartree_dims* dims, bool allow_split = true);
// record `msg` as this thread's dartree_last_error() and return `s`
dartree_status set_error(dartree_status s, const char* msg);

}  // namespace dartree
