// Fused per-head Q/K RMSNorm + partial three-axis MM-RoPE, in place, for gfx950.
//
// Operation ("MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 2 fingerprint
// rows "Q/K preprocessing", "Position encoding", "RoPE frequencies", "Rotary
// channels"; section 4 rule "Q/K RMSNorm happens before MM-RoPE", FP32
// frequency construction; section 5 items h3_qk_rmsnorm_d128 and
// h3_mm_rope_3axis_partial):
//   y_c = x_c / sqrt(mean(x^2) + 1e-5) * gamma_c          (one head row, 128 ch)
//   w_j = 1 / 10000^(2j/32), j = 0..15;  phi_{16a+j} = pos_a * w_j, a = t, h, w
//   for c < 48:  out_c = y_c cos phi_c - y_{c+48} sin phi_c
//                out_{c+48} = y_{c+48} cos phi_c + y_c sin phi_c
//   out_c = y_c for 96 <= c < 128;   one RNE rounding to bf16 at the end.
// Q's output may carry a scale factor q_scale (applied in fp32, folded into
// gamma_q, before that single rounding); q_scale = 1 leaves every bit as
// above.
//
// Memory-bound by construction: every Q and K head-row is read once (256 B)
// and written once, in place.  Mapping: one wave per token.  A quarter-wave
// (16 lanes) owns one 256-byte head-row; lane i < 12 holds the four rotation
// pairs (4i..4i+3, 48+4i..48+4i+3) so each pair sits inside one lane and the
// rotation needs no cross-lane traffic; lanes 12..15 hold pass-through
// channels 96..127.  The sum of squares is a 16-lane butterfly.  A lane's
// four angles depend only on the token, so their sines and cosines are
// computed once per token and reused for all 2H head-rows (Q then K) the wave
// walks through in chunks of kPasses 4-row passes whose loads are all in flight
// together; kPasses is chosen per H so the chunks waste the fewest row slots
// (14 passes = 56 rows for H = 56: each chunk is exactly one tensor's rows of
// the token).  A K-only form walks K's H rows alone and also stores each
// token's 48 cosines and sines, which the attention kernel's fused Q prologue
// reads instead of evaluating them again.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3attn {
namespace {

constexpr int kHeadDim = 128;
constexpr int kWavesPerBlock = 4;     // one token per wave

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x from lane (lane ^ m) of the same 16-lane row, m in {1, 2, 4, 8}, through
// the data-parallel-primitive lane selects of the vector ALU (no LDS round
// trip): quad permutes for m = 1, 2; a rotation by 8 within the row for m = 8;
// and for m = 4, a shift left by 4 into lane groups 0-3 and 8-11 and a shift
// right by 4 into lane groups 4-7 and 12-15 (the bank mask picks the groups).
template <int m>
__device__ __forceinline__ float row_xor(float x) {
  const int v = __float_as_int(x);
  int r;
  if (m == 1) r = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);        // quad_perm [1,0,3,2]
  else if (m == 2) r = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  else if (m == 8) r = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  else {
    r = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);   // row_shl:4 into groups 0, 2
    r = __builtin_amdgcn_update_dpp(r, v, 0x114, 0xF, 0xA, false);   // row_shr:4 into groups 1, 3
  }
  return __int_as_float(r);
}

// The sum over the 16 lanes of a row by the xor butterfly (1, 2, 4, 8): every
// lane ends with the same bits.
__device__ __forceinline__ float row_sum16(float x) {
  x += row_xor<1>(x);
  x += row_xor<2>(x);
  x += row_xor<4>(x);
  return x + row_xor<8>(x);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  r[0] = (__bf16)a;  // v_cvt_pk_bf16_f32: round to nearest even
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// FP8 form of K (the quantized-score path): byte position of channel c in a
// 128-byte k8 row.  The row is laid out as the attention kernel's FP8 score
// product reads it -- lane half g's 64 bytes first for g = 0, then g = 1, each
// two 32-byte k-steps of four 8-channel pieces -- so that a lane's operand is
// one contiguous read:  position 64 g + 32 s + 8 j + e holds channel
// 16 (4 s + j) + 8 g + e.
__device__ __forceinline__ int k8_position(int c) {
  return 64 * ((c >> 3) & 1) + 32 * (c >> 6) + 8 * ((c >> 4) & 3) + (c & 7);
}

// Four fp32 values -> four OCP FP8 e4m3 bytes (round to nearest even; the
// values here stay far inside the format's range).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// One wave's work: every head row of one token (Q's, then K's).  kKOnly:
// only K's rows, and the lane's cosines and sines go to rope_cs (fp32 [L][96]:
// cos of the token's 48 angles, then their sines) for an attention kernel that
// applies Q's prologue itself.  kK8 (with kKOnly): K's outputs, times 1/4, go to
// k8 as FP8 e4m3 (bytes ordered by k8_position) instead of back to k as bf16.
template <int kPassesPerChunk, bool kKOnly, bool kK8 = false>
__device__ __forceinline__ void prologue_token(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                               const float* __restrict__ gamma_q, const float* __restrict__ gamma_k,
                                               const int32_t* __restrict__ pos, int64_t token, int32_t H,
                                               float q_scale, float* __restrict__ rope_cs, int lane,
                                               uint8_t* __restrict__ k8 = nullptr) {
  static_assert(!kK8 || kKOnly, "the FP8 form is written for K alone");
  const int sub = lane >> 4;  // which of the pass's 4 rows this quarter-wave owns
  const int i = lane & 15;    // lane within the row
  const bool pair_lane = i < 12;
  // Channel offsets of the lane's two 4-channel pieces.
  const int ch_a = pair_lane ? 4 * i : 96 + 4 * (i - 12);
  const int ch_b = pair_lane ? 48 + 4 * i : 112 + 4 * (i - 12);

  float gqa[4], gqb[4], gka[4], gkb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gqa[e] = gamma_q[ch_a + e] * q_scale;
    gqb[e] = gamma_q[ch_b + e] * q_scale;
    gka[e] = gamma_k[ch_a + e];
    gkb[e] = gamma_k[ch_b + e];
  }

  // Angles of channels ch_a..ch_a+3 (pair lanes only): axis i/4, j = 4*(i%4) + e.
  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (pair_lane) {
    const float p = (float)pos[token * 3 + (i >> 2)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * (i & 3) + e;
      const float inv_freq = 1.0f / powf(10000.0f, (float)(2 * j) / 32.0f);
      sincosf(p * inv_freq, &sn[e], &cs[e]);
    }
    if (kKOnly && sub == 0) {  // angles 4i .. 4i+3 of the token
      *reinterpret_cast<float4*>(rope_cs + token * 96 + 4 * i) = make_float4(cs[0], cs[1], cs[2], cs[3]);
      *reinterpret_cast<float4*>(rope_cs + token * 96 + 48 + 4 * i) = make_float4(sn[0], sn[1], sn[2], sn[3]);
    }
  }

  const int rows = kKOnly ? H : 2 * H;  // Q rows 0..H-1, then K rows (K only: K rows 0..H-1)
  const int64_t token_base = token * (int64_t)H * kHeadDim;
  for (int r0 = 0; r0 < rows; r0 += 4 * kPassesPerChunk) {
    uint2 va[kPassesPerChunk], vb[kPassesPerChunk];
#pragma unroll
    for (int ps = 0; ps < kPassesPerChunk; ++ps) {
      const int rr = r0 + 4 * ps + sub;
      va[ps] = make_uint2(0u, 0u);
      vb[ps] = make_uint2(0u, 0u);
      if (rr < rows) {
        const bool rq = !kKOnly && rr < H;
        const uint16_t* row = (rq ? q : k) + token_base + (int64_t)(kKOnly || rq ? rr : rr - H) * kHeadDim;
        va[ps] = *reinterpret_cast<const uint2*>(row + ch_a);
        vb[ps] = *reinterpret_cast<const uint2*>(row + ch_b);
      }
    }
#pragma unroll
    for (int ps = 0; ps < kPassesPerChunk; ++ps) {
      const int rr = r0 + 4 * ps + sub;
      float xa[4] = {lo_bf16(va[ps].x), hi_bf16(va[ps].x), lo_bf16(va[ps].y), hi_bf16(va[ps].y)};
      float xb[4] = {lo_bf16(vb[ps].x), hi_bf16(vb[ps].x), lo_bf16(vb[ps].y), hi_bf16(vb[ps].y)};
      float ss = xa[0] * xa[0];
#pragma unroll
      for (int e = 1; e < 4; ++e) ss = fmaf(xa[e], xa[e], ss);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(xb[e], xb[e], ss);
      // Butterfly over the 16 lanes of the row: every lane ends with the same sum.
      ss = row_sum16(ss);
      const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + 1e-5f);
      const bool is_q = !kKOnly && rr < H;
      float oa[4], ob[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ya = xa[e] * r * (is_q ? gqa[e] : gka[e]);
        const float yb = xb[e] * r * (is_q ? gqb[e] : gkb[e]);
        oa[e] = fmaf(ya, cs[e], -(yb * sn[e]));
        ob[e] = fmaf(yb, cs[e], ya * sn[e]);
      }
      if (kK8 && rr < rows) {
        uint8_t* row8 = k8 + token_base + (int64_t)rr * kHeadDim;
        *reinterpret_cast<uint32_t*>(row8 + k8_position(ch_a)) =
            pack_e4m3x4(0.25f * oa[0], 0.25f * oa[1], 0.25f * oa[2], 0.25f * oa[3]);
        *reinterpret_cast<uint32_t*>(row8 + k8_position(ch_b)) =
            pack_e4m3x4(0.25f * ob[0], 0.25f * ob[1], 0.25f * ob[2], 0.25f * ob[3]);
      } else if (rr < rows) {
        uint16_t* row = (is_q ? q : k) + token_base + (int64_t)(kKOnly || is_q ? rr : rr - H) * kHeadDim;
        *reinterpret_cast<uint2*>(row + ch_a) = make_uint2(pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3]));
        *reinterpret_cast<uint2*>(row + ch_b) = make_uint2(pack_bf16x2(ob[0], ob[1]), pack_bf16x2(ob[2], ob[3]));
      }
    }
  }
}

template <int kPassesPerChunk, bool kKOnly>
__global__ __launch_bounds__(kWavesPerBlock * 64) void qk_prologue_kernel(
    uint16_t* __restrict__ q, uint16_t* __restrict__ k, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, const int32_t* __restrict__ pos, int64_t L, int32_t H,
    float q_scale, float* __restrict__ rope_cs) {
  const int64_t token = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (token >= L) return;  // whole wave exits together
  prologue_token<kPassesPerChunk, kKOnly>(q, k, gamma_q, gamma_k, pos, token, H, q_scale, rope_cs,
                                          threadIdx.x & 63);
}

// ---------------------------------------------------------------- V transpose
// vt[h][c][j] = v[j][h][c] for j < L, 0 for L <= j < Lp (Lp = L rounded up
// to 64): the layout the log2 attention kernels read V in.  One 256-thread
// workgroup per (64-key block, head): the block's 64 rows x 256 bytes go
// through LDS (row stride 65 words: the column reads then hit 32 distinct
// banks), and every 8 consecutive lanes write one 128-byte run of a V^T row.
constexpr int kVtThreads = 256;
constexpr int kVtKeys = 64;
constexpr int kVtTileWords = kVtKeys * 65;

__device__ __forceinline__ void v_transpose_tile(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt, int L,
                                                 int H, int Lp, int head, int key0, int tid, uint32_t* tile) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = i * kVtThreads + tid, r = idx >> 4, c16 = idx & 15;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (key0 + r < L)
      val = *reinterpret_cast<const uint4*>(v + ((int64_t)(key0 + r) * H + head) * kHeadDim + 8 * c16);
    uint32_t* dst = tile + r * 65 + 4 * c16;
    dst[0] = val.x;
    dst[1] = val.y;
    dst[2] = val.z;
    dst[3] = val.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = i * kVtThreads + tid, d = idx >> 3, c = idx & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[(8 * c + 2 * e) * 65 + (d >> 1)];
      const uint32_t hi = tile[(8 * c + 2 * e + 1) * 65 + (d >> 1)];
      w[e] = (d & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    *reinterpret_cast<uint4*>(vt + ((int64_t)head * kHeadDim + d) * Lp + key0 + 8 * c) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ __launch_bounds__(kVtThreads) void v_transpose_kernel(const uint16_t* __restrict__ v,
                                                                 uint16_t* __restrict__ vt, int L, int H,
                                                                 int Lp) {
  __shared__ uint32_t tile[kVtTileWords];
  const int nblk = Lp / kVtKeys;
  const int head = blockIdx.x / nblk, key0 = (blockIdx.x - head * nblk) * kVtKeys;
  v_transpose_tile(v, vt, L, H, Lp, head, key0, threadIdx.x, tile);
}

// ---------------------------------------------------------------- K prologue + V transpose
// One launch for the two passes the attention kernel with Q's prologue at its
// load needs before it runs: K's prologue in place with the rotation table
// (prologue_token, K only: the same bits as qk_prologue_kernel<P, true>) and
// V^T (v_transpose_tile: the same bits as v_transpose_kernel).  The two kinds
// of workgroup are dealt out in proportion, evenly over the grid (workgroup b
// does K work when floor((b + 1) nk / n) > floor(b nk / n)), so K's in-place
// traffic and V's read-and-scatter traffic share the memory system for the
// whole launch instead of running one after the other.
static_assert(kWavesPerBlock * 64 == kVtThreads, "both kinds of workgroup have 256 threads");

template <int kPassesPerChunk, bool kK8>
__global__ __launch_bounds__(kVtThreads) void kv_prologue_kernel(
    uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
    const float* __restrict__ gamma_k, const int32_t* __restrict__ pos, float* __restrict__ rope_cs, int64_t L,
    int32_t H, int Lp, int64_t nk, int64_t n, uint8_t* __restrict__ k8) {
  __shared__ uint32_t tile[kVtTileWords];
  const int64_t b = blockIdx.x;
  const int64_t kb = b * nk / n;
  if ((b + 1) * nk / n > kb) {
    const int64_t token = kb * kWavesPerBlock + (threadIdx.x >> 6);
    if (token < L)
      prologue_token<kPassesPerChunk, true, kK8>(nullptr, k, gamma_k, gamma_k, pos, token, H, 1.0f, rope_cs,
                                                 threadIdx.x & 63, k8);
    return;
  }
  const int64_t vb = b - kb;  // V workgroups before this one
  const int nblk = Lp / kVtKeys;
  const int head = (int)(vb / nblk), key0 = (int)(vb - (int64_t)head * nblk) * kVtKeys;
  v_transpose_tile(v, vt, (int)L, H, Lp, head, key0, threadIdx.x, tile);
}

// ---------------------------------------------------------------- backward
// Gradient of the prologue (same RFC, section 7, per-operator gate: forward
// and backward), for every row of Q and of K, given dy' = dLoss/d(output):
//   dy = inverse rotation of dy': for c < 48, dy_c = cos dy'_c + sin dy'_{c+48},
//        dy_{c+48} = cos dy'_{c+48} - sin dy'_c; dy_c = dy'_c for c >= 96
//   dx = r (gamma dy) - x r^3 mean(gamma dy x),  r = (mean(x^2) + eps)^(-1/2)
//   dgamma += dy x r   (summed over every token and head)
// x is the raw (pre-prologue) row; dx overwrites dy' in place (bf16, one RNE
// rounding).  Same mapping as the forward (one wave per token, a 16-lane
// quarter-wave per row, each rotation pair inside one lane).  The gamma
// gradients are summed without atomics: each lane keeps its channels' sums
// over the rows it handles, the workgroup adds its four waves in LDS in a
// fixed order and writes one partial per workgroup, and gamma_reduce_kernel
// adds those partials in a fixed order -- the result does not depend on timing.
__global__ __launch_bounds__(kWavesPerBlock * 64) void qk_prologue_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, const int32_t* __restrict__ pos, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, float* __restrict__ partial, int64_t L, int32_t H, float q_scale) {
  __shared__ float wsum[kWavesPerBlock][2 * kHeadDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t token = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const bool live = token < L;
  const int sub = lane >> 4, i = lane & 15;
  const bool pair_lane = i < 12;
  const int ch_a = pair_lane ? 4 * i : 96 + 4 * (i - 12);
  const int ch_b = pair_lane ? 48 + 4 * i : 112 + 4 * (i - 12);
  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (live && pair_lane) {
    const float p = (float)pos[token * 3 + (i >> 2)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * (i & 3) + e;
      const float inv_freq = 1.0f / powf(10000.0f, (float)(2 * j) / 32.0f);
      sincosf(p * inv_freq, &sn[e], &cs[e]);
    }
  }
  float gqa[4], gqb[4], gka[4], gkb[4];  // gammas at the lane's channels
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gqa[e] = gamma_q[ch_a + e] * q_scale;  // Q's effective weights, as in the forward
    gqb[e] = gamma_q[ch_b + e] * q_scale;
    gka[e] = gamma_k[ch_a + e];
    gkb[e] = gamma_k[ch_b + e];
  }
  float sqa[4] = {}, sqb[4] = {}, ska[4] = {}, skb[4] = {};  // this lane's dgamma sums
  const int64_t token_base = token * (int64_t)H * kHeadDim;
  const int rows = live ? 2 * H : 0;
  // kBwdRows rows per row group per pass, all loaded before any is computed (the
  // stores go to the buffers the next rows are read from, so the compiler would
  // not move those loads ahead of them); every row group runs the same passes.
  constexpr int kBwdRows = 4;
  const int rows_round = (rows + 4 * kBwdRows - 1) / (4 * kBwdRows) * (4 * kBwdRows);
  for (int base = 0; base < rows_round; base += 4 * kBwdRows) {
    uint2 xa[kBwdRows], xb[kBwdRows], da[kBwdRows], db[kBwdRows];
#pragma unroll
    for (int n = 0; n < kBwdRows; ++n) {
      const int rr = base + 4 * n + sub;
      xa[n] = xb[n] = da[n] = db[n] = make_uint2(0u, 0u);
      if (rr < rows) {
        const int t = rr < H ? 0 : 1;
        const int64_t off = token_base + (int64_t)(t == 0 ? rr : rr - H) * kHeadDim;
        const uint16_t* xr = (t == 0 ? q : k) + off;
        const uint16_t* dr = (t == 0 ? dq : dk) + off;
        xa[n] = *reinterpret_cast<const uint2*>(xr + ch_a);
        xb[n] = *reinterpret_cast<const uint2*>(xr + ch_b);
        da[n] = *reinterpret_cast<const uint2*>(dr + ch_a);
        db[n] = *reinterpret_cast<const uint2*>(dr + ch_b);
      }
    }
#pragma unroll
    for (int n = 0; n < kBwdRows; ++n) {
      const int rr = base + 4 * n + sub;
      const bool on = rr < rows;  // all 16 lanes of a row group share rr
      const int t = rr < H ? 0 : 1;
      const int64_t off = token_base + (int64_t)(t == 0 ? rr : rr - H) * kHeadDim;
      const float x_a[4] = {lo_bf16(xa[n].x), hi_bf16(xa[n].x), lo_bf16(xa[n].y), hi_bf16(xa[n].y)};
      const float x_b[4] = {lo_bf16(xb[n].x), hi_bf16(xb[n].x), lo_bf16(xb[n].y), hi_bf16(xb[n].y)};
      const float d_a[4] = {lo_bf16(da[n].x), hi_bf16(da[n].x), lo_bf16(da[n].y), hi_bf16(da[n].y)};
      const float d_b[4] = {lo_bf16(db[n].x), hi_bf16(db[n].x), lo_bf16(db[n].y), hi_bf16(db[n].y)};
      float ss = 0.f, tdot = 0.f, ya[4], yb[4], g_a[4], g_b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss = fmaf(x_a[e], x_a[e], ss);
        ss = fmaf(x_b[e], x_b[e], ss);
        ya[e] = fmaf(d_a[e], cs[e], d_b[e] * sn[e]);    // dy at ch_a (pass-through lanes: cs = 1, sn = 0)
        yb[e] = fmaf(d_b[e], cs[e], -(d_a[e] * sn[e]));  // dy at ch_b
        g_a[e] = (t == 0 ? gqa[e] : gka[e]) * ya[e];
        g_b[e] = (t == 0 ? gqb[e] : gkb[e]) * yb[e];
        tdot = fmaf(g_a[e], x_a[e], tdot);
        tdot = fmaf(g_b[e], x_b[e], tdot);
      }
      ss = row_sum16(ss);
      tdot = row_sum16(tdot);
      const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + 1e-5f);
      const float corr = r * r * r * tdot * (1.0f / kHeadDim);
      float oa[4], ob[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oa[e] = fmaf(r, g_a[e], -(x_a[e] * corr));
        ob[e] = fmaf(r, g_b[e], -(x_b[e] * corr));
        const float ua = on ? ya[e] * x_a[e] * r : 0.f, ub = on ? yb[e] * x_b[e] * r : 0.f;
        if (t == 0) {
          sqa[e] += ua;
          sqb[e] += ub;
        } else {
          ska[e] += ua;
          skb[e] += ub;
        }
      }
      if (on) {
        uint16_t* dr = (t == 0 ? dq : dk) + off;
        *reinterpret_cast<uint2*>(dr + ch_a) = make_uint2(pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3]));
        *reinterpret_cast<uint2*>(dr + ch_b) = make_uint2(pack_bf16x2(ob[0], ob[1]), pack_bf16x2(ob[2], ob[3]));
      }
    }
  }
  // The four row groups of the wave (lanes i, i+16, i+32, i+48), then the
  // workgroup's waves in order.
  auto group_sum = [](float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
  };
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sqa[e] = group_sum(sqa[e]);
    sqb[e] = group_sum(sqb[e]);
    ska[e] = group_sum(ska[e]);
    skb[e] = group_sum(skb[e]);
  }
  if (sub == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wsum[wave][ch_a + e] = sqa[e];
      wsum[wave][ch_b + e] = sqb[e];
      wsum[wave][kHeadDim + ch_a + e] = ska[e];
      wsum[wave][kHeadDim + ch_b + e] = skb[e];
    }
  }
  __syncthreads();
  const int c = threadIdx.x;  // 256 threads = 2 x 128 channels
  float acc = wsum[0][c];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) acc += wsum[w][c];
  partial[(int64_t)blockIdx.x * 2 * kHeadDim + c] = acc;
}

// out[j][c] = sum over rows j*32 .. j*32+31 (< n) of in[row][c], c < 256,
// rows added in increasing order.  All of a thread's loads are issued before
// the first add (a dependent chain of loads would leave the kernel waiting on
// memory latency row after row).
constexpr int kReduceRows = 32;

__global__ __launch_bounds__(2 * kHeadDim) void gamma_reduce_kernel(const float* __restrict__ in,
                                                                    float* __restrict__ out, int64_t n) {
  const int c = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kReduceRows;
  float x[kReduceRows];
#pragma unroll
  for (int i = 0; i < kReduceRows; ++i) x[i] = r0 + i < n ? in[(r0 + i) * 2 * kHeadDim + c] : 0.f;
  float acc = x[0];
#pragma unroll
  for (int i = 1; i < kReduceRows; ++i) acc += x[i];
  out[(int64_t)blockIdx.x * 2 * kHeadDim + c] = acc;
}

// The last stage: the n group sums, in order -> dgamma_q (c < 128, times
// q_scale: Q's output carried gamma_q * q_scale), dgamma_k; 16 loads in flight
// ahead of the adds.
__global__ __launch_bounds__(2 * kHeadDim) void gamma_final_kernel(const float* __restrict__ in, float* __restrict__ dgq,
                                                                   float* __restrict__ dgk, int64_t n, float q_scale) {
  const int c = threadIdx.x;
  float acc = 0.f;
  for (int64_t r0 = 0; r0 < n; r0 += 16) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = r0 + i < n ? in[(r0 + i) * 2 * kHeadDim + c] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (r0 + i < n) acc += x[i];
  }
  if (c < kHeadDim) dgq[c] = acc * q_scale;
  else dgk[c - kHeadDim] = acc;
}

}  // namespace

int64_t prologue_grid_blocks(int64_t L) { return (L + kWavesPerBlock - 1) / kWavesPerBlock; }

// Passes per chunk for n rows a token: the candidate whose chunks leave the
// fewest row slots empty, the larger on a tie.
static int prologue_passes(int64_t n) {
  const int candidates[3] = {14, 8, 4};
  int best = 14;
  int64_t best_waste = -1;
  for (int p : candidates) {
    const int64_t rows = 4 * p, waste = (n + rows - 1) / rows * rows - n;
    if (best_waste < 0 || waste < best_waste) best = p, best_waste = waste;
  }
  return best;
}

int64_t transpose_grid_blocks(int64_t L, int32_t H) { return vt_padded_length(L) / kVtKeys * (int64_t)H; }
int transpose_block_threads() { return kVtThreads; }
int64_t kv_prologue_grid_blocks(int64_t L, int32_t H) { return prologue_grid_blocks(L) + transpose_grid_blocks(L, H); }

hipError_t launch_v_transpose(const uint16_t* v, uint16_t* vt, int64_t L, int32_t H, hipStream_t stream) {
  hipLaunchKernelGGL(v_transpose_kernel, dim3((unsigned)transpose_grid_blocks(L, H)), dim3(kVtThreads), 0,
                     stream, v, vt, (int)L, (int)H, (int)vt_padded_length(L));
  return hipGetLastError();
}

template <bool kKOnly>
static void launch_prologue(uint16_t* q, uint16_t* k, const float* gamma_q, const float* gamma_k,
                            const int32_t* pos, int64_t L, int32_t H, float q_scale, float* rope_cs,
                            hipStream_t stream) {
  const dim3 grid((unsigned)prologue_grid_blocks(L)), block(kWavesPerBlock * 64);
  switch (prologue_passes(kKOnly ? H : 2 * (int64_t)H)) {
    case 14:
      hipLaunchKernelGGL((qk_prologue_kernel<14, kKOnly>), grid, block, 0, stream, q, k, gamma_q, gamma_k, pos, L,
                         H, q_scale, rope_cs);
      break;
    case 8:
      hipLaunchKernelGGL((qk_prologue_kernel<8, kKOnly>), grid, block, 0, stream, q, k, gamma_q, gamma_k, pos, L,
                         H, q_scale, rope_cs);
      break;
    default:
      hipLaunchKernelGGL((qk_prologue_kernel<4, kKOnly>), grid, block, 0, stream, q, k, gamma_q, gamma_k, pos, L,
                         H, q_scale, rope_cs);
      break;
  }
}

hipError_t launch_qk_prologue(uint16_t* q, uint16_t* k, const float* gamma_q, const float* gamma_k,
                              const int32_t* pos, int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  launch_prologue<false>(q, k, gamma_q, gamma_k, pos, L, H, q_scale, nullptr, stream);
  return hipGetLastError();
}

hipError_t launch_k_prologue(uint16_t* k, const float* gamma_k, const int32_t* pos, float* rope_cs, int64_t L,
                             int32_t H, hipStream_t stream) {
  launch_prologue<true>(nullptr, k, gamma_k, gamma_k, pos, L, H, 1.0f, rope_cs, stream);
  return hipGetLastError();
}

template <bool kK8>
static hipError_t launch_kv(uint16_t* k, const uint16_t* v, uint16_t* vt, const float* gamma_k, const int32_t* pos,
                            float* rope_cs, uint8_t* k8, int64_t L, int32_t H, hipStream_t stream) {
  const int64_t nk = prologue_grid_blocks(L), n = kv_prologue_grid_blocks(L, H);
  const int Lp = (int)vt_padded_length(L);
  const dim3 grid((unsigned)n), block(kVtThreads);
  switch (prologue_passes(H)) {
    case 14:
      hipLaunchKernelGGL((kv_prologue_kernel<14, kK8>), grid, block, 0, stream, k, v, vt, gamma_k, pos, rope_cs, L,
                         H, Lp, nk, n, k8);
      break;
    case 8:
      hipLaunchKernelGGL((kv_prologue_kernel<8, kK8>), grid, block, 0, stream, k, v, vt, gamma_k, pos, rope_cs, L,
                         H, Lp, nk, n, k8);
      break;
    default:
      hipLaunchKernelGGL((kv_prologue_kernel<4, kK8>), grid, block, 0, stream, k, v, vt, gamma_k, pos, rope_cs, L,
                         H, Lp, nk, n, k8);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_kv_prologue(uint16_t* k, const uint16_t* v, uint16_t* vt, const float* gamma_k, const int32_t* pos,
                              float* rope_cs, int64_t L, int32_t H, hipStream_t stream) {
  return launch_kv<false>(k, v, vt, gamma_k, pos, rope_cs, nullptr, L, H, stream);
}

hipError_t launch_kv_prologue_fp8(const uint16_t* k, const uint16_t* v, uint16_t* vt, const float* gamma_k,
                                  const int32_t* pos, float* rope_cs, uint8_t* k8, int64_t L, int32_t H,
                                  hipStream_t stream) {
  return launch_kv<true>(const_cast<uint16_t*>(k), v, vt, gamma_k, pos, rope_cs, k8, L, H, stream);
}

// Workspace of the backward: one 256-float partial per workgroup, then one per
// 256 of those.
static int64_t bwd_blocks(int64_t L) { return prologue_grid_blocks(L); }
static int64_t bwd_groups(int64_t L) { return (bwd_blocks(L) + kReduceRows - 1) / kReduceRows; }

int64_t prologue_backward_workspace_bytes(int64_t L) {
  return (bwd_blocks(L) + bwd_groups(L)) * 2 * kHeadDim * (int64_t)sizeof(float);
}

hipError_t launch_qk_prologue_backward(const uint16_t* q, const uint16_t* k, const float* gamma_q,
                                       const float* gamma_k, const int32_t* pos, uint16_t* dq, uint16_t* dk,
                                       float* dgamma_q, float* dgamma_k, float* workspace, int64_t L, int32_t H,
                                       float q_scale, hipStream_t stream) {
  const int64_t nb = bwd_blocks(L), ng = bwd_groups(L);
  float* partial = workspace;
  float* groups = workspace + nb * 2 * kHeadDim;
  hipLaunchKernelGGL(qk_prologue_bwd_kernel, dim3((unsigned)nb), dim3(kWavesPerBlock * 64), 0, stream, q, k,
                     gamma_q, gamma_k, pos, dq, dk, partial, L, H, q_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gamma_reduce_kernel, dim3((unsigned)ng), dim3(2 * kHeadDim), 0, stream, partial, groups, nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gamma_final_kernel, dim3(1), dim3(2 * kHeadDim), 0, stream, groups, dgamma_q, dgamma_k, ng,
                     q_scale);
  return hipGetLastError();
}

}  // namespace h3attn
