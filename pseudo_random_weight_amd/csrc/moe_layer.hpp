// The routed MoE layer of seedmm.hip, shared with the other sources of the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/seedmm.h"

namespace seedmm_layer {

// The routed layer (arguments, results and errors of seedmm_moe).  P = 3 or 4 for one P,
// or P = 0 with p4mask (device, bit e set = expert e has P = 4) for mixed packs, whose
// expert kernels run once per P.  events: NULL or 5 hipEvent_t recorded between the
// stages.  slot: NULL, or device int32[E] giving the slot of expert e (an expert cache):
// the streams of slot s start s * slot_stride bytes after gate/up/down's pointers; every
// routed expert must have a valid slot.  side: NULL, or the caller's second stream and
// fork / join events (seedmm_moe_ex).
int moe_run(const int32_t* topk_ids, const float* topk_w, int T, int top_k, const void* x,
            float* y, int E, int H, int I, int P, const uint32_t* p4mask, seedmm_mat gate,
            seedmm_mat up, seedmm_mat down, void* workspace, size_t workspace_bytes,
            void* hip_stream, void* const* events, const int32_t* slot,
            int64_t slot_stride, const seedmm_side* side);

}  // namespace seedmm_layer
