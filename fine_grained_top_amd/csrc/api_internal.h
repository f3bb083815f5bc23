// Entry-point plumbing shared by the C-ABI source files: the forward
// attention call split into validation and launch, so entry points that
// differ only in where the workspace comes from share both.
#pragma once
#include <stddef.h>

#include "../../include/spattn.h"
#include "internal.h"

namespace spapi {

// Records msg as the thread's last error message and returns code.
int set_error(int code, const char* msg);
// SPATTN_OK when the current HIP device is a usable gfx950.
int device_check();
// Validates a forward attention call (no HIP call) and fills p; need gets the
// workspace bytes the launch will use.
int attn_fwd_prepare(const spattn_tensor* q, const spattn_tensor* k, const spattn_tensor* v,
                     const spattn_kv_pages* pages, const int32_t* ctx_len, float scale, const spattn_selection* sel,
                     const spattn_tensor* o_out, float* lse_out, sp::AttnParams& p, size_t& need);
// Checks the device and enqueues the attention kernels with workspace ws.
int attn_fwd_launch(sp::AttnParams& p, void* ws, size_t ws_bytes, void* stream);

}  // namespace spapi
