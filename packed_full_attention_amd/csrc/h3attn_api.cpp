// C ABI of libh3attn: argument validation, then one kernel launch per call.
//
// Validation is synchronous, happens before any HIP call and rejects instead of
// falling back (fail closed: "MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 4
// item 9 and section 7 "Per-operator gate": empty, mis-shaped or unsupported
// inputs fail clearly).  Device contents are never inspected.
#include "h3attn.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "h3attn_internal.h"

namespace {

thread_local char g_last_error[256];

int fail(int status, const char* fmt, const char* detail = nullptr) {
  snprintf(g_last_error, sizeof g_last_error, fmt, detail ? detail : "");
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return H3A_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Do the byte ranges [a, a+na) and [b, b+nb) overlap?
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr int64_t kMaxThreadsPerGrid = (int64_t)1 << 32;  // work-items per grid dimension

// Common shape checks; on success *bytes is the size of one [L][H][128] bf16 tensor.
int check_shape(int64_t L, int32_t H, uint64_t* bytes) {
  if (L <= 0) return fail(H3A_EINVAL, "L must be >= 1 (empty documents are rejected)%s");
  if (H <= 0) return fail(H3A_EINVAL, "H must be >= 1%s");
  if (L >= ((int64_t)1 << 31)) return fail(H3A_EUNSUPPORTED, "L must be < 2^31%s");
  const __int128 elems = (__int128)L * H * H3ATTN_HEAD_DIM;
  if (elems * 2 > ((__int128)1 << 62)) return fail(H3A_EUNSUPPORTED, "L*H*128 too large%s");
  *bytes = (uint64_t)(elems * 2);
  return H3A_OK;
}

// The attention kernels address a tile through a buffer resource with 32-bit
// per-lane byte offsets (and a 32-bit size), so every byte a tile DMA reads must
// lie within 2^32 - 1 bytes of the tile's first byte; past that the offsets
// would wrap and read other rows.  Such geometries are rejected.
constexpr int64_t kMaxTileSpan = 0xffffffffLL;

int check_row_tiles(int32_t H) {
  if (h3attn::row_tile_dma_end(H) > kMaxTileSpan || h3attn::backward_tile_dma_end(H) > kMaxTileSpan)
    return fail(H3A_EUNSUPPORTED, "H too large: a 64-token tile of [L][H][128] spans more than 2^32 bytes%s");
  return H3A_OK;
}

int check_vt_tiles(int64_t L) {
  if (h3attn::vt_tile_dma_end(L) > kMaxTileSpan)
    return fail(H3A_EUNSUPPORTED, "L too large for vt: a 64-key tile of [H][128][Lp] spans more than 2^32 bytes%s");
  return H3A_OK;
}

// The prologue kernels count a token's 2H head rows (Q's, then K's) in 32-bit
// integers, in steps of up to 64 rows.
int check_prologue_rows(int32_t H) {
  if (2 * (int64_t)H + 64 > INT32_MAX) return fail(H3A_EUNSUPPORTED, "H too large for the prologue (2H + 64 >= 2^31)%s");
  return H3A_OK;
}

}  // namespace

extern "C" {

int h3attn_abi_version(void) { return H3ATTN_ABI_VERSION; }

const char* h3attn_strerror(int status) {
  switch (status) {
    case H3A_OK: return "success";
    case H3A_EINVAL: return "invalid argument";
    case H3A_EUNSUPPORTED: return "unsupported geometry";
    case H3A_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* h3attn_last_error(void) { return g_last_error; }

namespace {

int prologue(void* q, void* k, const float* gamma_q, const float* gamma_k, const int32_t* pos_thw, int64_t L,
             int32_t H, float q_scale, hipStream_t stream) {
  if (!q || !k || !gamma_q || !gamma_k || !pos_thw)
    return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(q, 16) || !aligned(k, 16)) return fail(H3A_EINVAL, "q and k must be 16-byte aligned%s");
  if (!aligned(gamma_q, 4) || !aligned(gamma_k, 4) || !aligned(pos_thw, 4))
    return fail(H3A_EINVAL, "gamma_q, gamma_k and pos_thw must be 4-byte aligned%s");
  if (!(isfinite(q_scale) && q_scale > 0.0f)) return fail(H3A_EINVAL, "q_scale must be finite and > 0%s");
  if (overlap(q, bytes, k, bytes)) return fail(H3A_EINVAL, "q and k overlap%s");
  // q and k are rewritten while the weights and positions are read.
  const uint64_t pbytes = (uint64_t)L * 12;
  for (const void* w : {q, k})
    if (overlap(w, bytes, gamma_q, 512) || overlap(w, bytes, gamma_k, 512) || overlap(w, bytes, pos_thw, pbytes))
      return fail(H3A_EINVAL, "q or k overlaps gamma_q, gamma_k or pos_thw%s");
  if (h3attn::prologue_grid_blocks(L) * 256 >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "prologue grid too large for L%s");
  if (int s = check_prologue_rows(H)) return s;
  const hipError_t e = h3attn::launch_qk_prologue(static_cast<uint16_t*>(q), static_cast<uint16_t*>(k),
                                                  gamma_q, gamma_k, pos_thw, L, H, q_scale, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}

int forward(const void* q, const void* k, const void* v, void* out, int64_t L, int32_t H, float scale,
            bool log2, hipStream_t stream, float* lse = nullptr) {
  if (!q || !k || !v || !out) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(H3A_EINVAL, log2 ? "q, k, vt and out must be 16-byte aligned%s"
                                 : "q, k, v and out must be 16-byte aligned%s");
  if (!(isfinite(scale) && scale > 0.0f)) return fail(H3A_EINVAL, "scale must be finite and > 0%s");
  const uint64_t vbytes = log2 ? (uint64_t)h3attn::vt_bytes(L, H) : bytes;
  if (overlap(out, bytes, q, bytes) || overlap(out, bytes, k, bytes) || overlap(out, bytes, v, vbytes))
    return fail(H3A_EINVAL, log2 ? "out overlaps q, k or vt%s" : "out overlaps q, k or v%s");
  if (lse != nullptr) {
    const uint64_t lbytes = (uint64_t)L * H * 4;
    if (!aligned(lse, 4)) return fail(H3A_EINVAL, "lse must be 4-byte aligned%s");
    if (overlap(lse, lbytes, q, bytes) || overlap(lse, lbytes, k, bytes) || overlap(lse, lbytes, v, vbytes) ||
        overlap(lse, lbytes, out, bytes))
      return fail(H3A_EINVAL, "lse overlaps q, k, v or out%s");
  }
  if (h3attn::attention_grid_blocks(L, H) * h3attn::attention_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "attention grid too large for (L, H)%s");
  if (int s = check_row_tiles(H)) return s;
  if (log2)
    if (int s = check_vt_tiles(L)) return s;
  const hipError_t e = h3attn::launch_attention_forward(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(out), lse, L, H, scale, log2, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

int64_t h3attn_vt_bytes(int64_t L, int32_t H) {
  uint64_t bytes = 0;
  if (check_shape(L, H, &bytes) != H3A_OK) return -1;
  ok();
  return h3attn::vt_bytes(L, H);
}

int h3attn_v_transpose(const void* v, void* vt, int64_t L, int32_t H, hipStream_t stream) {
  if (!v || !vt) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(v, 16) || !aligned(vt, 16)) return fail(H3A_EINVAL, "v and vt must be 16-byte aligned%s");
  if (overlap(vt, (uint64_t)h3attn::vt_bytes(L, H), v, bytes)) return fail(H3A_EINVAL, "vt overlaps v%s");
  if (h3attn::transpose_grid_blocks(L, H) * h3attn::transpose_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "transpose grid too large for (L, H)%s");
  const hipError_t e = h3attn::launch_v_transpose(static_cast<const uint16_t*>(v), static_cast<uint16_t*>(vt), L,
                                                  H, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "transpose launch failed: %s", hipGetErrorString(e));
  return ok();
}

int h3attn_qk_prologue(void* q, void* k, const float* gamma_q, const float* gamma_k,
                       const int32_t* pos_thw, int64_t L, int32_t H, hipStream_t stream) {
  return prologue(q, k, gamma_q, gamma_k, pos_thw, L, H, 1.0f, stream);
}

int h3attn_qk_prologue_scaled(void* q, void* k, const float* gamma_q, const float* gamma_k,
                              const int32_t* pos_thw, int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  return prologue(q, k, gamma_q, gamma_k, pos_thw, L, H, q_scale, stream);
}

int h3attn_forward(const void* q, const void* k, const void* v, void* out, int64_t L, int32_t H,
                   float scale, hipStream_t stream) {
  return forward(q, k, v, out, L, H, scale, false, stream);
}

int h3attn_forward_log2(const void* q, const void* k, const void* vt, void* out, int64_t L, int32_t H,
                        hipStream_t stream) {
  return forward(q, k, vt, out, L, H, 1.0f, true, stream);
}

int h3attn_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int64_t L,
                       int32_t H, float scale, hipStream_t stream) {
  if (!lse) return fail(H3A_EINVAL, "null pointer argument%s");
  return forward(q, k, v, out, L, H, scale, false, stream, lse);
}

int h3attn_forward_log2_lse(const void* q, const void* k, const void* vt, void* out, float* lse, int64_t L,
                            int32_t H, hipStream_t stream) {
  if (!lse) return fail(H3A_EINVAL, "null pointer argument%s");
  return forward(q, k, vt, out, L, H, 1.0f, true, stream, lse);
}

int64_t h3attn_rope_table_bytes(int64_t L, int32_t H) {
  uint64_t bytes = 0;
  if (check_shape(L, H, &bytes) != H3A_OK) return -1;
  ok();
  return L * 96 * 4;
}

int h3attn_k_prologue_table(void* k, const float* gamma_k, const int32_t* pos_thw, float* rope_cs, int64_t L,
                            int32_t H, hipStream_t stream) {
  if (!k || !gamma_k || !pos_thw || !rope_cs) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(k, 16) || !aligned(rope_cs, 16)) return fail(H3A_EINVAL, "k and rope_cs must be 16-byte aligned%s");
  if (!aligned(gamma_k, 4) || !aligned(pos_thw, 4))
    return fail(H3A_EINVAL, "gamma_k and pos_thw must be 4-byte aligned%s");
  const uint64_t tbytes = (uint64_t)L * 96 * 4;
  if (overlap(rope_cs, tbytes, k, bytes) || overlap(rope_cs, tbytes, gamma_k, 512) ||
      overlap(rope_cs, tbytes, pos_thw, (uint64_t)L * 12))
    return fail(H3A_EINVAL, "rope_cs overlaps k, gamma_k or pos_thw%s");
  if (overlap(k, bytes, gamma_k, 512) || overlap(k, bytes, pos_thw, (uint64_t)L * 12))
    return fail(H3A_EINVAL, "k overlaps gamma_k or pos_thw%s");
  if (h3attn::prologue_grid_blocks(L) * 256 >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "prologue grid too large for L%s");
  if (int s = check_prologue_rows(H)) return s;
  const hipError_t e =
      h3attn::launch_k_prologue(static_cast<uint16_t*>(k), gamma_k, pos_thw, rope_cs, L, H, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}

int h3attn_kv_prologue(void* k, const void* v, const float* gamma_k, const int32_t* pos_thw, float* rope_cs, void* vt,
                       int64_t L, int32_t H, hipStream_t stream) {
  if (!k || !v || !gamma_k || !pos_thw || !rope_cs || !vt) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(rope_cs, 16) || !aligned(vt, 16))
    return fail(H3A_EINVAL, "k, v, rope_cs and vt must be 16-byte aligned%s");
  if (!aligned(gamma_k, 4) || !aligned(pos_thw, 4))
    return fail(H3A_EINVAL, "gamma_k and pos_thw must be 4-byte aligned%s");
  // Written: k (in place), rope_cs, vt; read: v, gamma_k, pos_thw (and k).
  const uint64_t tbytes = (uint64_t)L * 96 * 4, vtb = (uint64_t)h3attn::vt_bytes(L, H), pbytes = (uint64_t)L * 12;
  const void* wr[3] = {k, rope_cs, vt};
  const uint64_t wn[3] = {bytes, tbytes, vtb};
  const void* in[3] = {v, gamma_k, pos_thw};
  const uint64_t inn[3] = {bytes, 512, pbytes};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(wr[i], wn[i], in[j], inn[j])) return fail(H3A_EINVAL, "k, rope_cs or vt overlaps v, gamma_k or pos_thw%s");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(wr[i], wn[i], wr[j], wn[j])) return fail(H3A_EINVAL, "k, rope_cs and vt overlap%s");
  }
  if (h3attn::kv_prologue_grid_blocks(L, H) * h3attn::transpose_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "prologue grid too large for (L, H)%s");
  if (int s = check_prologue_rows(H)) return s;
  const hipError_t e = h3attn::launch_kv_prologue(static_cast<uint16_t*>(k), static_cast<const uint16_t*>(v),
                                                  static_cast<uint16_t*>(vt), gamma_k, pos_thw, rope_cs, L, H, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}

int h3attn_kv_prologue_fp8(const void* k, const void* v, const float* gamma_k, const int32_t* pos_thw,
                           float* rope_cs, void* k8, void* vt, int64_t L, int32_t H, hipStream_t stream) {
  if (!k || !v || !gamma_k || !pos_thw || !rope_cs || !k8 || !vt) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(rope_cs, 16) || !aligned(vt, 16) || !aligned(k8, 16))
    return fail(H3A_EINVAL, "k, v, rope_cs, k8 and vt must be 16-byte aligned%s");
  if (!aligned(gamma_k, 4) || !aligned(pos_thw, 4))
    return fail(H3A_EINVAL, "gamma_k and pos_thw must be 4-byte aligned%s");
  // Written: rope_cs, k8, vt; read: k, v, gamma_k, pos_thw.
  const uint64_t tbytes = (uint64_t)L * 96 * 4, vtb = (uint64_t)h3attn::vt_bytes(L, H), pbytes = (uint64_t)L * 12;
  const void* wr[3] = {rope_cs, k8, vt};
  const uint64_t wn[3] = {tbytes, bytes / 2, vtb};
  const void* in[4] = {k, v, gamma_k, pos_thw};
  const uint64_t inn[4] = {bytes, bytes, 512, pbytes};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(wr[i], wn[i], in[j], inn[j]))
        return fail(H3A_EINVAL, "rope_cs, k8 or vt overlaps k, v, gamma_k or pos_thw%s");
    for (int j = i + 1; j < 3; ++j)
      if (overlap(wr[i], wn[i], wr[j], wn[j])) return fail(H3A_EINVAL, "rope_cs, k8 and vt overlap%s");
  }
  if (h3attn::kv_prologue_grid_blocks(L, H) * h3attn::transpose_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "prologue grid too large for (L, H)%s");
  if (int s = check_prologue_rows(H)) return s;
  const hipError_t e = h3attn::launch_kv_prologue_fp8(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                                      static_cast<uint16_t*>(vt), gamma_k, pos_thw, rope_cs,
                                                      static_cast<uint8_t*>(k8), L, H, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}

int h3attn_forward_fp8_qprologue(const void* q, const void* k8, const void* vt, void* out, const float* gamma_q,
                                 const float* rope_cs, int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  if (!q || !k8 || !vt || !out || !gamma_q || !rope_cs) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(q, 16) || !aligned(k8, 16) || !aligned(vt, 16) || !aligned(out, 16) || !aligned(gamma_q, 16) ||
      !aligned(rope_cs, 16))
    return fail(H3A_EINVAL, "q, k8, vt, out, gamma_q and rope_cs must be 16-byte aligned%s");
  if (!(isfinite(q_scale) && q_scale > 0.0f)) return fail(H3A_EINVAL, "q_scale must be finite and > 0%s");
  const uint64_t vbytes = (uint64_t)h3attn::vt_bytes(L, H), tbytes = (uint64_t)L * 96 * 4;
  if (overlap(out, bytes, q, bytes) || overlap(out, bytes, k8, bytes / 2) || overlap(out, bytes, vt, vbytes) ||
      overlap(out, bytes, gamma_q, 512) || overlap(out, bytes, rope_cs, tbytes))
    return fail(H3A_EINVAL, "out overlaps q, k8, vt, gamma_q or rope_cs%s");
  if (h3attn::attention_grid_blocks(L, H) * h3attn::attention_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "attention grid too large for (L, H)%s");
  if (int s = check_row_tiles(H)) return s;
  if (int s = check_vt_tiles(L)) return s;
  const hipError_t e = h3attn::launch_attention_forward_fp8(
      static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k8), static_cast<const uint16_t*>(vt),
      static_cast<uint16_t*>(out), gamma_q, rope_cs, L, H, q_scale, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

int h3attn_forward_log2_qprologue(const void* q, const void* k, const void* vt, void* out, const float* gamma_q,
                                  const float* rope_cs, int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  if (!q || !k || !vt || !out || !gamma_q || !rope_cs) return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vt, 16) || !aligned(out, 16) || !aligned(gamma_q, 16) ||
      !aligned(rope_cs, 16))
    return fail(H3A_EINVAL, "q, k, vt, out, gamma_q and rope_cs must be 16-byte aligned%s");
  if (!(isfinite(q_scale) && q_scale > 0.0f)) return fail(H3A_EINVAL, "q_scale must be finite and > 0%s");
  const uint64_t vbytes = (uint64_t)h3attn::vt_bytes(L, H), tbytes = (uint64_t)L * 96 * 4;
  if (overlap(out, bytes, q, bytes) || overlap(out, bytes, k, bytes) || overlap(out, bytes, vt, vbytes) ||
      overlap(out, bytes, gamma_q, 512) || overlap(out, bytes, rope_cs, tbytes))
    return fail(H3A_EINVAL, "out overlaps q, k, vt, gamma_q or rope_cs%s");
  if (h3attn::attention_grid_blocks(L, H) * h3attn::attention_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "attention grid too large for (L, H)%s");
  if (int s = check_row_tiles(H)) return s;
  if (int s = check_vt_tiles(L)) return s;
  const hipError_t e = h3attn::launch_attention_forward_qprologue(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(vt),
      static_cast<uint16_t*>(out), gamma_q, rope_cs, L, H, q_scale, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

int64_t h3attn_attention_backward_workspace_bytes(int64_t L, int32_t H) {
  uint64_t bytes = 0;
  if (check_shape(L, H, &bytes) != H3A_OK) return -1;
  ok();
  return h3attn::backward_workspace_bytes(L, H);
}

namespace {

// Validation shared by the two forms of the attention backward; workspace may
// be null for the form that holds its statistics in the library (ws_bytes 0).
int check_attention_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, void* workspace, uint64_t ws_bytes,
                             int64_t L, int32_t H, float scale) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || (ws_bytes && !workspace))
    return fail(H3A_EINVAL, "null pointer argument%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  const void* bf[8] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : bf)
    if (!aligned(p, 16)) return fail(H3A_EINVAL, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned%s");
  if (!aligned(lse, 4) || !aligned(workspace, 4)) return fail(H3A_EINVAL, "lse and workspace must be 4-byte aligned%s");
  if (!(isfinite(scale) && scale > 0.0f)) return fail(H3A_EINVAL, "scale must be finite and > 0%s");
  const uint64_t vec = (uint64_t)L * H * 4;
  // Written ranges: dq, dk, dv, workspace; none may meet another or any input.
  const void* wr[4] = {dq, dk, dv, workspace};
  const uint64_t wn[4] = {bytes, bytes, bytes, ws_bytes};
  const void* in[6] = {q, k, v, out, dout, lse};
  const uint64_t inn[6] = {bytes, bytes, bytes, bytes, bytes, vec};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(wr[i], wn[i], in[j], inn[j])) return fail(H3A_EINVAL, "an output or the workspace overlaps an input%s");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(wr[i], wn[i], wr[j], wn[j])) return fail(H3A_EINVAL, "outputs or workspace overlap%s");
  }
  if (h3attn::backward_grid_blocks(L, H) * h3attn::backward_block_threads() >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "backward grid too large for (L, H)%s");
  if (int s = check_row_tiles(H)) return s;
  return H3A_OK;
}

int launch_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, float* stats, int64_t L, int32_t H, float scale, hipStream_t stream) {
  const hipError_t e = h3attn::launch_attention_backward(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), lse, static_cast<uint16_t*>(dq),
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), stats, L, H, scale, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

int h3attn_attention_backward(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              void* workspace, int64_t L, int32_t H, float scale, hipStream_t stream) {
  uint64_t bytes = 0;
  const uint64_t ws = check_shape(L, H, &bytes) == H3A_OK ? (uint64_t)h3attn::backward_workspace_bytes(L, H) : 1;
  if (int s = check_attention_backward(q, k, v, out, dout, lse, dq, dk, dv, workspace, ws, L, H, scale)) return s;
  return launch_backward(q, k, v, out, dout, lse, dq, dk, dv, static_cast<float*>(workspace), L, H, scale, stream);
}

int h3attn_attention_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                      const void* dout, const float* lse, void* dq, void* dk, void* dv, int64_t L,
                                      int32_t H, float scale, hipStream_t stream) {
  if (int s = check_attention_backward(q, k, v, out, dout, lse, dq, dk, dv, nullptr, 0, L, H, scale)) return s;
  if (h3attn::backward_workspace_bytes(L, H) > h3attn::backward_static_scratch_bytes())
    return fail(H3A_EUNSUPPORTED, "(L, H) too large for the library's scratch: needs H * Lp <= 2^21 "
                                  "(Lp = L rounded up to 64)%s");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(H3A_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(H3A_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev) return fail(H3A_EINVAL, "stream belongs to a device other than the current one%s");
  }
  float* stats = nullptr;
  e = h3attn::backward_static_scratch(dev, &stats);
  if (e != hipSuccess) return fail(H3A_EHIP, "scratch lookup failed: %s", hipGetErrorString(e));
  return launch_backward(q, k, v, out, dout, lse, dq, dk, dv, stats, L, H, scale, stream);
}

int64_t h3attn_qk_prologue_backward_workspace_bytes(int64_t L, int32_t H) {
  uint64_t bytes = 0;
  if (check_shape(L, H, &bytes) != H3A_OK) return -1;
  ok();
  return h3attn::prologue_backward_workspace_bytes(L);
}

namespace {

int prologue_backward(const void* q, const void* k, const float* gamma_q, const float* gamma_k,
                      const int32_t* pos_thw, void* dq, void* dk, float* dgamma_q, float* dgamma_k, void* workspace,
                      int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  if (!q || !k || !gamma_q || !gamma_k || !pos_thw || !dq || !dk || !dgamma_q || !dgamma_k || !workspace)
    return fail(H3A_EINVAL, "null pointer argument%s");
  if (!(isfinite(q_scale) && q_scale > 0.0f)) return fail(H3A_EINVAL, "q_scale must be finite and > 0%s");
  uint64_t bytes = 0;
  if (int s = check_shape(L, H, &bytes)) return s;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(dq, 16) || !aligned(dk, 16))
    return fail(H3A_EINVAL, "q, k, dq and dk must be 16-byte aligned%s");
  if (!aligned(gamma_q, 4) || !aligned(gamma_k, 4) || !aligned(pos_thw, 4) || !aligned(dgamma_q, 4) ||
      !aligned(dgamma_k, 4) || !aligned(workspace, 4))
    return fail(H3A_EINVAL, "gammas, positions, gamma gradients and workspace must be 4-byte aligned%s");
  const uint64_t ws = (uint64_t)h3attn::prologue_backward_workspace_bytes(L);
  const void* wr[5] = {dq, dk, dgamma_q, dgamma_k, workspace};
  const uint64_t wn[5] = {bytes, bytes, 512, 512, ws};
  const void* in[5] = {q, k, gamma_q, gamma_k, pos_thw};
  const uint64_t inn[5] = {bytes, bytes, 512, 512, (uint64_t)L * 12};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(wr[i], wn[i], in[j], inn[j])) return fail(H3A_EINVAL, "an output or the workspace overlaps an input%s");
    for (int j = i + 1; j < 5; ++j)
      if (overlap(wr[i], wn[i], wr[j], wn[j])) return fail(H3A_EINVAL, "outputs or workspace overlap%s");
  }
  if (h3attn::prologue_grid_blocks(L) * 256 >= kMaxThreadsPerGrid)
    return fail(H3A_EUNSUPPORTED, "prologue grid too large for L%s");
  if (int s = check_prologue_rows(H)) return s;
  const hipError_t e = h3attn::launch_qk_prologue_backward(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), gamma_q, gamma_k, pos_thw,
      static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk), dgamma_q, dgamma_k, static_cast<float*>(workspace), L,
      H, q_scale, stream);
  if (e != hipSuccess) return fail(H3A_EHIP, "prologue backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

int h3attn_qk_prologue_backward(const void* q, const void* k, const float* gamma_q, const float* gamma_k,
                                const int32_t* pos_thw, void* dq, void* dk, float* dgamma_q,
                                float* dgamma_k, void* workspace, int64_t L, int32_t H,
                                hipStream_t stream) {
  return prologue_backward(q, k, gamma_q, gamma_k, pos_thw, dq, dk, dgamma_q, dgamma_k, workspace, L, H, 1.0f,
                           stream);
}

int h3attn_qk_prologue_backward_scaled(const void* q, const void* k, const float* gamma_q, const float* gamma_k,
                                       const int32_t* pos_thw, void* dq, void* dk, float* dgamma_q,
                                       float* dgamma_k, void* workspace, int64_t L, int32_t H, float q_scale,
                                       hipStream_t stream) {
  return prologue_backward(q, k, gamma_q, gamma_k, pos_thw, dq, dk, dgamma_q, dgamma_k, workspace, L, H, q_scale,
                           stream);
}

}  // extern "C"
