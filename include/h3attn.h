/*
 * h3attn -- packed full attention for the MiniMax-H3 Omni-Transformer block on
 * AMD Instinct MI355X (gfx950).  Plain C ABI, no C++ or torch types.
 *
 * The path: per-head Q/K RMSNorm -> partial three-axis MM-RoPE (both in
 * h3attn_qk_prologue) -> full bidirectional softmax(Q K^T * scale) V
 * (h3attn_forward), over one packed text + video + audio document.
 *
 * Definitions are those of the "MiniMax-H3 WS1/WS2 kernel roadmap" RFC:
 *   section 2, Omni-Transformer fingerprint table (56 heads x 128, full
 *   bidirectional self-attention, per-head Q/K RMSNorm with epsilon 1e-5,
 *   three-axis (t, h, w) MM-RoPE with 16 frequencies per axis, theta 10000,
 *   96 of 128 channels rotated and 32 passed through);
 *   section 4, numerical contract (norm before RoPE, FP32 frequency
 *   construction, non-causal unmasked attention over one document, fixed
 *   reduction order, no split-KV or atomics, fail closed on unsupported input);
 *   section 5, work items h3_qk_rmsnorm_d128, h3_mm_rope_3axis_partial and
 *   h3_full_attention.
 *
 * Common conventions
 *   - Tensors q, k, v, out are bfloat16 (raw 16-bit patterns), contiguous,
 *     token-major [L][H][128]: element (l, h, c) sits at ((l*H + h)*128 + c).
 *     Batch is not an argument: a batch is a replication axis, so callers
 *     issue one call per document.
 *   - All pointers are device memory owned by the caller.  The library
 *     allocates nothing and only enqueues work on `stream` (0 = the null
 *     stream): the calls return before the GPU finishes, and the caller
 *     synchronises.  Between calls it keeps only the text of the calling
 *     thread's last error (h3attn_last_error, thread-local) and, for
 *     h3attn_attention_backward_noalloc alone, a device array per device
 *     (its address, looked up once, and whatever the last such call left in
 *     it).
 *   - Arguments are validated on the host before any launch; a rejected call
 *     launches nothing and leaves every buffer untouched.  There is no
 *     fallback path.  Device data is not inspected: non-finite inputs
 *     propagate, and positions must satisfy |pos| <= 2^24 (exact in fp32).
 *   - Results are deterministic: a fixed key order and one workgroup per
 *     output row, independent of launch geometry, so repeated calls are
 *     bit-identical, and a query row's output (a key row's dk, dv) does not
 *     depend on where in the launch the row falls.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3ATTN_ABI_VERSION 8
#define H3ATTN_HEAD_DIM 128

/* Status codes. */
#define H3A_OK 0            /* success (work enqueued)                               */
#define H3A_EINVAL 1        /* null pointer, L <= 0, H <= 0, misalignment, overlap,   */
                            /* or a non-finite / non-positive scale or q_scale        */
#define H3A_EUNSUPPORTED 2  /* geometry outside the supported range: L >= 2^31, a    */
                            /* grid or size overflow, or a tile whose bytes span more */
                            /* than 2^32 (the attention calls need 63*H*256 + 256 <=  */
                            /* 2^32 - 1; the vt calls 254*Lp + 128 <= 2^32 - 1; the   */
                            /* prologue calls 2H + 64 < 2^31)                         */
#define H3A_EHIP 3          /* the HIP launch reported an error                       */

/*
 * Q/K prologue, in place: for every token l and head h,
 *   q[l,h,:] <- RoPE_pos[l]( RMSNorm_gamma_q( q[l,h,:] ) )
 *   k[l,h,:] <- RoPE_pos[l]( RMSNorm_gamma_k( k[l,h,:] ) )
 * RMSNorm: y_c = x_c / sqrt(mean_c(x_c^2) + 1e-5) * gamma_c over the 128
 * channels of one head, evaluated in fp32.
 * MM-RoPE: with w_j = 10000^(-j/16) (j = 0..15, fp32) and angles
 * phi_{16a+j} = pos[l,a] * w_j for axes a = t, h, w, channel c < 48 and its
 * partner c + 48 rotate by phi_c:
 *   out_c    = y_c * cos(phi_c) - y_{c+48} * sin(phi_c)
 *   out_{c+48} = y_{c+48} * cos(phi_c) + y_c * sin(phi_c)
 * and channels 96..127 pass through.  One round-to-nearest-even to bf16 at
 * the end; accurate fp32 sine and cosine.
 *
 *   q, k     bf16 [L][H][128], read and rewritten in place; 16-byte aligned;
 *            the two ranges must not overlap each other or gamma_q, gamma_k,
 *            pos_thw.
 *   gamma_q, gamma_k  fp32 [128] RMSNorm weights, shared by all heads;
 *            4-byte aligned.
 *   pos_thw  int32 [L][3] per-token (t, h, w) positions; 4-byte aligned.
 *   L        tokens in the packed document, 1 <= L < 2^31.
 *   H        heads, >= 1.
 */
int h3attn_qk_prologue(void* q, void* k, const float* gamma_q, const float* gamma_k,
                       const int32_t* pos_thw, int64_t L, int32_t H, hipStream_t stream);

/*
 * Full bidirectional attention, per head h, over all L tokens with no mask:
 *   out[i,h,:] = sum_j softmax_j( scale * <q[i,h,:], k[j,h,:]> ) * v[j,h,:]
 * S = Q K^T and P V on bf16 matrix cores with fp32 accumulation; online
 * softmax in fp32 (P rounded to bf16 as the P V operand); the output is
 * divided by the fp32 row sum and rounded to bf16 (round to nearest even).
 *
 *   q, k, v  bf16 [L][H][128] inputs (q and k normally come from
 *            h3attn_qk_prologue; v is used as given); 16-byte aligned; they
 *            may alias one another.
 *   out      bf16 [L][H][128] output; 16-byte aligned; must not overlap q, k
 *            or v.
 *   L, H     as above.
 *   scale    softmax scale, finite and > 0 (1/sqrt(128) for the H3 block).
 */
int h3attn_forward(const void* q, const void* k, const void* v, void* out, int64_t L,
                   int32_t H, float scale, hipStream_t stream);

/*
 * The same path in the layout the fastest kernel reads.  Together,
 *   h3attn_qk_prologue_scaled(q, k, gamma_q, gamma_k, pos_thw, L, H, scale * log2(e), s)
 *   h3attn_v_transpose(v, vt, L, H, s)
 *   h3attn_forward_log2(q, k, vt, out, L, H, s)
 * compute what h3attn_qk_prologue + h3attn_forward(..., scale, s) compute, with
 * the same single bf16 rounding of q (of the scaled values instead of the
 * unscaled ones).  The attention kernel then evaluates each exponential
 * straight from the matrix-core score, without a scaling instruction per score,
 * and reads every P V operand from the transposed V in one 16-byte LDS read.
 *
 * h3attn_qk_prologue_scaled: as h3attn_qk_prologue, except that the Q output
 *   is multiplied by q_scale (finite, > 0; applied in fp32 before the rounding
 *   to bf16).  q_scale = 1 gives h3attn_qk_prologue's output bit for bit.
 *
 * h3attn_vt_bytes: the size of vt for (L, H): H * 128 * Lp * 2 bytes with
 *   Lp = L rounded up to a multiple of 64; -1 for an (L, H) the other calls
 *   reject (L <= 0, H <= 0, L >= 2^31, too large).
 *
 * h3attn_v_transpose: vt[h][c][j] = v[j][h][c] for j < L and 0 for
 *   L <= j < Lp: bf16 [H][128][Lp], caller-owned device memory of
 *   h3attn_vt_bytes(L, H) bytes, 16-byte aligned, not overlapping v.  A pure
 *   copy (bit exact).
 *
 * h3attn_forward_log2: base-2 softmax attention, per head h,
 *   out[i,h,:] = sum_j 2^<q[i,h,:], k[j,h,:]> v[j,h,:] / sum_j 2^<q[i,h,:], k[j,h,:]>
 *   i.e. h3attn_forward with scale = ln 2 (and so, with q from
 *   h3attn_qk_prologue_scaled at q_scale = scale * log2(e), the scale-`scale`
 *   attention of the unscaled q), with V given as vt from h3attn_v_transpose
 *   (its padding columns must be zero).  q, k, out as for h3attn_forward; out
 *   must not overlap q, k or vt.
 */
int h3attn_qk_prologue_scaled(void* q, void* k, const float* gamma_q, const float* gamma_k,
                              const int32_t* pos_thw, int64_t L, int32_t H, float q_scale,
                              hipStream_t stream);
int64_t h3attn_vt_bytes(int64_t L, int32_t H);
int h3attn_v_transpose(const void* v, void* vt, int64_t L, int32_t H, hipStream_t stream);
int h3attn_forward_log2(const void* q, const void* k, const void* vt, void* out, int64_t L,
                        int32_t H, hipStream_t stream);

/*
 * The same path with Q's prologue fused into the attention kernel's Q load,
 * as the "h3-metal" README ("Implementation and performance notes",
 * "Profiling and diagnostic paths") fuses Q/K RMS normalization and RoPE into
 * the kernel that produces Q and K, with byte-identical results.  Together,
 *   h3attn_k_prologue_table(k, gamma_k, pos_thw, rope_cs, L, H, s)
 *   h3attn_v_transpose(v, vt, L, H, s)
 *   h3attn_forward_log2_qprologue(q, k, vt, out, gamma_q, rope_cs, L, H, q_scale, s)
 * give the same out, bit for bit, as h3attn_qk_prologue_scaled(..., q_scale,
 * s) + h3attn_v_transpose + h3attn_forward_log2, and the same k; q is only
 * read.  Q's prologue output never goes to memory (one write and one read of
 * Q fewer), and its rotation reuses the per-token table K's prologue writes.
 *
 * h3attn_rope_table_bytes: L * 96 * 4 (-1 for an (L, H) the calls reject).
 *
 * h3attn_k_prologue_table: h3attn_qk_prologue on k alone (in place, same
 *   bits), and rope_cs[l][a] = cos(phi_a), rope_cs[l][48 + a] = sin(phi_a)
 *   for the 48 angles phi_a of token l (fp32 [L][96], as the prologue
 *   evaluates them).  rope_cs: caller-owned device memory of
 *   h3attn_rope_table_bytes(L, H) bytes, 16-byte aligned; k, rope_cs, gamma_k
 *   and pos_thw must not overlap.
 *
 * h3attn_forward_log2_qprologue: h3attn_forward_log2 of q' = the scaled
 *   prologue of the raw q (as h3attn_qk_prologue_scaled computes it with
 *   gamma_q, the positions behind rope_cs and q_scale), k from
 *   h3attn_k_prologue_table, vt from h3attn_v_transpose.  q: raw bf16
 *   [L][H][128], not modified; gamma_q fp32 [128] and rope_cs 16-byte
 *   aligned; q_scale finite and > 0 (scale * log2(e) for softmax scale
 *   `scale`); out must not overlap q, k, vt, gamma_q or rope_cs.
 */
/*
 * h3attn_kv_prologue: h3attn_k_prologue_table(k, gamma_k, pos_thw, rope_cs, L, H, s)
 *   and h3attn_v_transpose(v, vt, L, H, s) in one launch, with the same results
 *   bit for bit (k rewritten in place, rope_cs fp32 [L][96], vt bf16
 *   [H][128][Lp]): the two memory-bound passes the fused attention call needs,
 *   their traffic spread over one grid.  k, v, rope_cs, vt 16-byte aligned;
 *   gamma_k, pos_thw 4-byte aligned; k, rope_cs and vt must not overlap one
 *   another or v, gamma_k, pos_thw.
 */
int h3attn_kv_prologue(void* k, const void* v, const float* gamma_k, const int32_t* pos_thw, float* rope_cs,
                       void* vt, int64_t L, int32_t H, hipStream_t stream);

/*
 * Quantized-score variant (the "next" item of a quantized QK^T attention in the
 * spirit of the SageAttention baseline the "H3 Parity Evidence Ledger" page
 * names; MiniMax-H3 WS1/WS2 kernel roadmap RFC, section 4: a split or cast
 * outside the contract must be declared): the scores are computed from Q' and K'
 * rounded to OCP FP8 e4m3 (round to nearest even) on the FP8 matrix
 * instruction, everything else as the scale-folded fused path.  Its output is
 * NOT the bf16 path's: it follows
 *   out = softmax_2( e4m3(4 q') e4m3(k'/4)^T ) v,   softmax_2(s)_j = 2^s_j / sum 2^s
 * with q' = q_scale * prologue(q) and k' = prologue(k) evaluated in fp32, and
 * carries e4m3's 3-bit mantissa in every score term (about 3-4% relative L2
 * against the exact attention on ordinary inputs, much more where a few keys
 * dominate).  Use it where that accuracy is declared acceptable.
 *
 * h3attn_kv_prologue_fp8: as h3attn_kv_prologue (rope_cs and vt the same bits),
 *   but K's prologue output, divided by 4, goes to k8 as e4m3 bytes instead of
 *   back to k: k8 is caller-owned, L * H * 128 bytes, 16-byte aligned, one
 *   128-byte row per (token, head) with its channels in the order the attention
 *   kernel reads them (byte 64 g + 32 s + 8 j + e holds channel
 *   16 (4 s + j) + 8 g + e); k is read only.  rope_cs, k8 and vt must not overlap
 *   one another or k, v, gamma_k, pos_thw.
 *
 * h3attn_forward_fp8_qprologue: attention of the raw q (Q's prologue with
 *   gamma_q, the rope_cs table and q_scale applied at the load, then times 4 and
 *   rounded to e4m3) against k8 and vt from h3attn_kv_prologue_fp8; q_scale =
 *   scale * log2(e) for softmax scale `scale`.  Arguments as for
 *   h3attn_forward_log2_qprologue, with k8 in place of k.  Precondition (device
 *   data, not checked): |4 q'| and |k'/4| below 448, the largest e4m3 value
 *   (prologue outputs are at most sqrt(128) max|gamma| in magnitude).
 */
int h3attn_kv_prologue_fp8(const void* k, const void* v, const float* gamma_k, const int32_t* pos_thw,
                           float* rope_cs, void* k8, void* vt, int64_t L, int32_t H, hipStream_t stream);
int h3attn_forward_fp8_qprologue(const void* q, const void* k8, const void* vt, void* out, const float* gamma_q,
                                 const float* rope_cs, int64_t L, int32_t H, float q_scale, hipStream_t stream);

int64_t h3attn_rope_table_bytes(int64_t L, int32_t H);
int h3attn_k_prologue_table(void* k, const float* gamma_k, const int32_t* pos_thw, float* rope_cs,
                            int64_t L, int32_t H, hipStream_t stream);
int h3attn_forward_log2_qprologue(const void* q, const void* k, const void* vt, void* out,
                                  const float* gamma_q, const float* rope_cs, int64_t L, int32_t H,
                                  float q_scale, hipStream_t stream);

/*
 * Training: the backward pass ("MiniMax-H3 WS1/WS2 kernel roadmap" RFC,
 * section 7, per-operator gate: forward and backward of each operator).
 *
 * h3attn_forward_lse: h3attn_forward, and in addition
 *   lse[h*L + i] = ln( sum_j exp( scale * <q[i,h,:], k[j,h,:]> ) )
 *   fp32 [H][L], 4-byte aligned, not overlapping q, k, v or out.
 *
 * h3attn_attention_backward: given dout = dLoss/dout of that forward, with
 *   P = softmax(scale Q K^T) per head (recomputed from lse), O = out,
 *     dv = P^T dout
 *     dS = P * (dout V^T - delta),  delta_i = <dout_i, out_i>
 *     dq = scale dS K,  dk = scale dS^T Q
 *   q, k, v, out, dout: bf16 [L][H][128] (q, k as passed to the forward,
 *   i.e. after the prologue); lse: that forward's lse; dq, dk, dv: bf16
 *   [L][H][128] outputs (fp32 accumulation, one rounding); workspace:
 *   caller-owned device memory of h3attn_attention_backward_workspace_bytes(L, H)
 *   bytes (it receives per-row statistics: -lse log2(e) and -delta, fp32
 *   [2][H][Lp], Lp = L rounded up to a multiple of 64).  All 16-byte aligned (lse, the
 *   workspace: 4); the outputs and the workspace must not overlap one another
 *   or any input.  Two launches on `stream`; deterministic (no atomics, no
 *   split: one wave produces each output row).
 *
 * h3attn_qk_prologue_backward: given dq, dk = the gradients with respect to
 *   the prologue's outputs, overwrites them (in place) with the gradients with
 *   respect to its inputs q, k, and writes the gamma gradients:
 *     dy = inverse rotation of the output gradient (RoPE^T)
 *     dx = r (gamma dy) - x r^3 mean(gamma dy x),  r = (mean(x^2) + 1e-5)^(-1/2)
 *     dgamma[c] = sum over every token and head of dy_c x_c r
 *   q, k: the prologue's raw inputs (bf16 [L][H][128], not modified; keep a
 *   copy, since h3attn_qk_prologue rewrites them); gamma_q, gamma_k, pos_thw
 *   as for h3attn_qk_prologue; dq, dk bf16 [L][H][128], in place; dgamma_q,
 *   dgamma_k fp32 [128]; workspace: h3attn_qk_prologue_backward_workspace_bytes(L, H)
 *   bytes.  The gamma sums are added in a fixed order (deterministic).
 *
 * The *_workspace_bytes calls return -1 for an (L, H) the others reject.
 *
 * The training step in the scale-folded layout (c = fp32(scale * log2(e))):
 *   h3attn_qk_prologue_scaled(q, k, ..., c, s)            q' = c * prologue(q)
 *   h3attn_v_transpose(v, vt, L, H, s)
 *   h3attn_forward_log2_lse(q', k, vt, out, lse, L, H, s)
 *   h3attn_attention_backward(q', k, v, out, dout, lse, dq', dk, dv, ws, L, H, ln 2, s)
 *   h3attn_qk_prologue_backward_scaled(q, k, ..., dq', dk, ..., c, s)
 * gives the gradients of the plain path: ln 2 * <q', k> is the scaled score,
 * so the attention backward at scale ln 2 returns dk, dv and the gradient with
 * respect to q', which the scaled prologue backward carries back to the raw q.
 *
 * h3attn_forward_log2_lse: h3attn_forward_log2, and in addition
 *   lse[h*L + i] = ln( sum_j 2^<q[i,h,:], k[j,h,:]> )  (= ln sum_j exp(scale <q_raw', k>)
 *   for q = c * q_raw'), fp32 [H][L], as for h3attn_forward_lse.
 *
 * h3attn_qk_prologue_backward_scaled: h3attn_qk_prologue_backward for the
 *   prologue that h3attn_qk_prologue_scaled computed with this q_scale (finite,
 *   > 0): dq holds the gradient with respect to Q's scaled output, Q's weights
 *   are gamma_q * q_scale (fp32) and dgamma_q is q_scale * sum(dy x r).  With
 *   q_scale = 1 it is h3attn_qk_prologue_backward, bit for bit.
 */
int h3attn_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int64_t L,
                       int32_t H, float scale, hipStream_t stream);
int64_t h3attn_attention_backward_workspace_bytes(int64_t L, int32_t H);
int h3attn_attention_backward(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              void* workspace, int64_t L, int32_t H, float scale, hipStream_t stream);
int h3attn_forward_log2_lse(const void* q, const void* k, const void* vt, void* out, float* lse, int64_t L,
                            int32_t H, hipStream_t stream);
int64_t h3attn_qk_prologue_backward_workspace_bytes(int64_t L, int32_t H);
int h3attn_qk_prologue_backward(const void* q, const void* k, const float* gamma_q, const float* gamma_k,
                                const int32_t* pos_thw, void* dq, void* dk, float* dgamma_q,
                                float* dgamma_k, void* workspace, int64_t L, int32_t H,
                                hipStream_t stream);
int h3attn_qk_prologue_backward_scaled(const void* q, const void* k, const float* gamma_q,
                                       const float* gamma_k, const int32_t* pos_thw, void* dq, void* dk,
                                       float* dgamma_q, float* dgamma_k, void* workspace, int64_t L,
                                       int32_t H, float q_scale, hipStream_t stream);

/*
 * For callers that cannot allocate memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation -- and so cannot provide the
 * workspace: h3attn_attention_backward with its per-row statistics held in the
 * library's own device array (16 MiB on each device that loads the library,
 * kept until the process ends) instead of a caller workspace.  Same arguments
 * without the workspace, same kernels, same results bit for bit.
 *   Limit: H * Lp <= 2^21 (Lp = L rounded up to a multiple of 64; at H = 56,
 *   L <= 37440); larger (L, H) return H3A_EUNSUPPORTED before any launch.
 *   `stream` must belong to the calling thread's current device (else
 *   H3A_EINVAL).  The call allocates nothing; the first call on a device looks
 *   up that device's array (hipGetSymbolAddress).
 *   All calls on one device share its array: two of these calls whose work
 *   overlaps on one device (different streams, no ordering between them) race
 *   and may give wrong gradients.  Calls ordered on one stream are safe.
 */
int h3attn_attention_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                      int64_t L, int32_t H, float scale, hipStream_t stream);

/* Static description of a status code. */
const char* h3attn_strerror(int status);

/*
 * Detail of the last failed call on the calling thread (which argument was
 * rejected, or the HIP error string); "" when the last call succeeded.
 * The pointer stays valid until the next h3attn call on the same thread.
 */
const char* h3attn_last_error(void);

/* H3ATTN_ABI_VERSION of the built library. */
int h3attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
