// Host entry points of the balanced split (pa_decode_balanced.hip) used by
// the decode entry points in pa_decode.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// Ranges the balanced split's workspace must hold for these sizes.
int64_t balanced_split_ranges(int num_seqs, int hq, int max_len);

// Workspace bytes of the balanced split for `ranges` ranges.
size_t balanced_split_workspace_bytes(int hq, int head_dim, int64_t ranges);

// Plan, decode and merge of the balanced split on `st` (bf16/fp16, head_dim 64
// or 128); `ws` holds balanced_split_workspace_bytes(hq, head_dim, ranges).
pa_status launch_balanced_split(pa_dtype dtype, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* tables, const int32_t* lens,
                                float scale_log2, void* out, int num_seqs, int hq, int hkv,
                                int head_dim, int max_blocks, int64_t ranges, char* ws,
                                hipStream_t st);

}  // namespace pa
