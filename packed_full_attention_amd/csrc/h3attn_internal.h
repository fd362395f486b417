// Internal launch entry points shared by the C ABI layer and the kernel files.
// Arguments are already validated by the caller (h3attn_api.cpp).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace h3attn {

// Enqueue the fused Q/K RMSNorm + MM-RoPE kernel (in place on q and k).
hipError_t launch_qk_prologue(uint16_t* q, uint16_t* k, const float* gamma_q,
                              const float* gamma_k, const int32_t* pos, int64_t L, int32_t H,
                              hipStream_t stream);

// Enqueue the attention forward: the V transpose into the workspace vt, then
// the flash-attention kernel.
hipError_t launch_attention_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, uint16_t* vt, int64_t L, int32_t H, float scale,
                                    hipStream_t stream);

// Bytes of the forward's workspace (V^T, [H][128][L rounded up to 64], bf16).
int64_t attention_workspace_bytes(int64_t L, int32_t H);

// Grid sizes (workgroups) and workgroup sizes (threads) of the launches for
// (L, H); used by validation.
int64_t attention_grid_blocks(int64_t L, int32_t H);
int attention_block_threads();
int64_t transpose_grid_blocks(int64_t L, int32_t H);
int transpose_block_threads();
int64_t prologue_grid_blocks(int64_t L);

}  // namespace h3attn
