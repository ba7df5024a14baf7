// Host-side entry points of the kernel translation units (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_common.h"

namespace sdpa18 {

// Query rows per workgroup of each kernel family (the grid is
// ceil(Sq / block_m) x B x Hq workgroups).
int fp8_block_m(int d);
int fp8_pp_block_m();
int f32_block_m();
int bf16_block_m(int d);
int bf16_pp_block_m();

// bf16 inputs and output; d in {64, 128}.
hipError_t launch_attn_bf16(const AttnParams& p, int d, bool causal, hipStream_t stream);

// bf16, d = 128: eight waves in matrix-core / vector-unit ping-pong.
hipError_t launch_attn_bf16_pp(const AttnParams& p, bool causal, hipStream_t stream);

// fp8-e4m3fn inputs, bf16 output; d in {64, 128} (d = 128 runs the eight-wave
// ping-pong kernel).
hipError_t launch_attn_fp8(const AttnParams& p, int d, bool causal, hipStream_t stream);

// fp8-e4m3fn inputs, bf16 output, d = 128: eight waves in ping-pong.
hipError_t launch_attn_fp8_pp(const AttnParams& p, bool causal, hipStream_t stream);

// fp32 inputs and output; d in {64, 128}.
hipError_t launch_attn_f32(const AttnParams& p, int d, bool causal, hipStream_t stream);

}  // namespace sdpa18
