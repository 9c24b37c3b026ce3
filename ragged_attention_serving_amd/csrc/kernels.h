// Launchers for the gfx950 kernels (each defined next to its kernel).
#pragma once

#include <hip/hip_runtime.h>

#include "params.h"

namespace xattn {

// fp32 storage and arithmetic, any mask, head_dim 16/32/64/128; units of <= 4 rows.
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);
// bf16 decode: units of up to `rows` query rows sharing one KV head (rows in 1,2,4,8).
hipError_t launch_attn_decode(const AttnParams& p, int rows, hipStream_t stream);
// bf16 MFMA tiles: units of up to 128 query rows sharing one KV head.
hipError_t launch_attn_mma(const AttnParams& p, hipStream_t stream);
// log-sum-exp merge of split rows into out (dtype 0 fp32, 1 bf16) and lse.
hipError_t launch_merge(const AttnParams& p, int dtype, hipStream_t stream);

}  // namespace xattn
