// Internal launch entry points shared by the C ABI layer and the kernel files.
// Arguments are already validated by the caller (h3attn_api.cpp).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace h3attn {

// Enqueue the fused Q/K RMSNorm + MM-RoPE kernel (in place on q and k); Q's
// output is multiplied by q_scale before its rounding to bf16.
hipError_t launch_qk_prologue(uint16_t* q, uint16_t* k, const float* gamma_q,
                              const float* gamma_k, const int32_t* pos, int64_t L, int32_t H,
                              float q_scale, hipStream_t stream);

// The prologue on K alone (in place), plus each token's rotation table
// rope_cs ([L][96] fp32: cos of angles 0..47, then their sines).
hipError_t launch_k_prologue(uint16_t* k, const float* gamma_k, const int32_t* pos, float* rope_cs, int64_t L,
                             int32_t H, hipStream_t stream);

// Enqueue the flash-attention forward kernel.  log2 = false: weights
// exp(scale <q,k>), v row-major [L][H][128]; log2 = true: weights 2^<q,k>
// (q already carries the softmax scale times log2(e)), scale ignored, and v
// is V^T as written by launch_v_transpose.  lse (may be null): fp32 [H][L],
// each row's natural log-sum-exp of its scaled scores.
hipError_t launch_attention_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, float* lse, int64_t L, int32_t H, float scale, bool log2,
                                    hipStream_t stream);

// The log2 variant with Q's prologue applied at its Q load: q_raw holds the
// raw rows, gamma_q (16-byte aligned) and rope_cs ([L][96] fp32, as written by
// launch_k_prologue) supply the RMSNorm weights and the rotation; q_scale as
// in launch_qk_prologue.  Same result bits as launch_qk_prologue followed by
// the log2 variant.
hipError_t launch_attention_forward_qprologue(const uint16_t* q_raw, const uint16_t* k, const uint16_t* vt,
                                              uint16_t* out, const float* gamma_q, const float* rope_cs,
                                              int64_t L, int32_t H, float q_scale, hipStream_t stream);

// The quantized-score variant: Q's prologue at the load as above, its output
// times 4 rounded to FP8 e4m3, scores against k8 (h3attn_kv_prologue_fp8's FP8
// K, k'/4) on the FP8 matrix instruction; softmax and P V as the log2 variant.
hipError_t launch_attention_forward_fp8(const uint16_t* q_raw, const uint8_t* k8, const uint16_t* vt, uint16_t* out,
                                        const float* gamma_q, const float* rope_cs, int64_t L, int32_t H,
                                        float q_scale, hipStream_t stream);

// Enqueue the attention backward (two kernels, in this order): dq and the
// per-row statistics -lse log2(e) and -delta = -<dout, out> (stats, fp32
// [2][H][Lp], Lp = L rounded up to 64; written), then dk and dv.  q, k are
// the prologue outputs, lse the forward's [H][L] log-sum-exp.
hipError_t launch_attention_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* out, const uint16_t* dout, const float* lse,
                                     uint16_t* dq, uint16_t* dk, uint16_t* dv, float* stats, int64_t L,
                                     int32_t H, float scale, hipStream_t stream);
int64_t backward_grid_blocks(int64_t L, int32_t H);
int64_t backward_workspace_bytes(int64_t L, int32_t H);
int backward_block_threads();
int64_t backward_tile_dma_end(int32_t H);

// The library's own statistics buffer for the attention backward, one copy per
// device, of backward_static_scratch_bytes() bytes: its device address on
// device dev (which must be the current device; looked up on the first call
// per device and kept).
int64_t backward_static_scratch_bytes();
hipError_t backward_static_scratch(int dev, float** ptr);

// Backward of the prologue (in place on dq, dk) and the gamma gradients;
// workspace of prologue_backward_workspace_bytes(L) bytes.  q_scale: the
// factor launch_qk_prologue applied to Q's output (dq is the gradient with
// respect to that scaled output).
hipError_t launch_qk_prologue_backward(const uint16_t* q, const uint16_t* k, const float* gamma_q,
                                       const float* gamma_k, const int32_t* pos, uint16_t* dq, uint16_t* dk,
                                       float* dgamma_q, float* dgamma_k, float* workspace, int64_t L, int32_t H,
                                       float q_scale, hipStream_t stream);
int64_t prologue_backward_workspace_bytes(int64_t L);

// V^T = [H][128][Lp] bf16, Lp = L rounded up to 64, zeros past L.
hipError_t launch_v_transpose(const uint16_t* v, uint16_t* vt, int64_t L, int32_t H, hipStream_t stream);

// launch_k_prologue and launch_v_transpose in one launch (same results, bit
// for bit); its grid size for validation.
hipError_t launch_kv_prologue(uint16_t* k, const uint16_t* v, uint16_t* vt, const float* gamma_k, const int32_t* pos,
                              float* rope_cs, int64_t L, int32_t H, hipStream_t stream);
int64_t kv_prologue_grid_blocks(int64_t L, int32_t H);

// launch_kv_prologue with K's prologue output written as FP8 e4m3 to k8
// (bytes [L][H][128], each value k'/4, channels ordered as the FP8 attention
// kernel reads them) instead of back to k (read only).
hipError_t launch_kv_prologue_fp8(const uint16_t* k, const uint16_t* v, uint16_t* vt, const float* gamma_k,
                                  const int32_t* pos, float* rope_cs, uint8_t* k8, int64_t L, int32_t H,
                                  hipStream_t stream);
int64_t vt_padded_length(int64_t L);
int64_t vt_bytes(int64_t L, int32_t H);
int64_t transpose_grid_blocks(int64_t L, int32_t H);
int transpose_block_threads();

// An upper bound on the grid size (workgroups) of a forward launch for (L, H),
// its workgroup size (threads), and the prologue's grid size; used by
// validation (no HIP call).
int64_t attention_grid_blocks(int64_t L, int32_t H);
// How many of the last full 256-row q-tiles a forward or dq launch runs as two
// 128-row workgroups (to fill the grid's last round); results do not depend
// on it.
int forward_half_tiles(int64_t L, int32_t H);
int attention_block_threads();
int64_t prologue_grid_blocks(int64_t L);

// The tile DMA of the attention kernels addresses a tile through a buffer
// resource with 32-bit per-lane offsets: these give one past the last byte a
// row-major tile ([L][H][128], 64 rows) or a V^T tile (128 channel rows of 64
// keys) reads, counted from the tile's first byte.  Validation rejects any
// geometry where that end exceeds 2^32 - 1.
int64_t row_tile_dma_end(int32_t H);
int64_t vt_tile_dma_end(int64_t L);

}  // namespace h3attn
