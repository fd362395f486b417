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
// the token).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3attn {
namespace {

constexpr int kHeadDim = 128;
constexpr int kWavesPerBlock = 4;     // one token per wave

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  r[0] = (__bf16)a;  // v_cvt_pk_bf16_f32: round to nearest even
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

template <int kPassesPerChunk>
__global__ __launch_bounds__(kWavesPerBlock * 64) void qk_prologue_kernel(
    uint16_t* __restrict__ q, uint16_t* __restrict__ k, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, const int32_t* __restrict__ pos, int64_t L, int32_t H,
    float q_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t token = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (token >= L) return;  // whole wave exits together

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
  }

  const int rows = 2 * H;  // Q rows 0..H-1, then K rows
  const int64_t token_base = token * (int64_t)H * kHeadDim;
  for (int r0 = 0; r0 < rows; r0 += 4 * kPassesPerChunk) {
    uint2 va[kPassesPerChunk], vb[kPassesPerChunk];
#pragma unroll
    for (int ps = 0; ps < kPassesPerChunk; ++ps) {
      const int rr = r0 + 4 * ps + sub;
      va[ps] = make_uint2(0u, 0u);
      vb[ps] = make_uint2(0u, 0u);
      if (rr < rows) {
        const uint16_t* row = (rr < H ? q : k) + token_base + (int64_t)(rr < H ? rr : rr - H) * kHeadDim;
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
      ss += __shfl_xor(ss, 1, 16);
      ss += __shfl_xor(ss, 2, 16);
      ss += __shfl_xor(ss, 4, 16);
      ss += __shfl_xor(ss, 8, 16);
      const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + 1e-5f);
      const bool is_q = rr < H;
      float oa[4], ob[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ya = xa[e] * r * (is_q ? gqa[e] : gka[e]);
        const float yb = xb[e] * r * (is_q ? gqb[e] : gkb[e]);
        oa[e] = fmaf(ya, cs[e], -(yb * sn[e]));
        ob[e] = fmaf(yb, cs[e], ya * sn[e]);
      }
      if (rr < rows) {
        uint16_t* row = (is_q ? q : k) + token_base + (int64_t)(is_q ? rr : rr - H) * kHeadDim;
        *reinterpret_cast<uint2*>(row + ch_a) = make_uint2(pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3]));
        *reinterpret_cast<uint2*>(row + ch_b) = make_uint2(pack_bf16x2(ob[0], ob[1]), pack_bf16x2(ob[2], ob[3]));
      }
    }
  }
}

}  // namespace

int64_t prologue_grid_blocks(int64_t L) { return (L + kWavesPerBlock - 1) / kWavesPerBlock; }

// Passes per chunk for 2H rows: the candidate whose chunks leave the fewest
// row slots empty, the larger on a tie.
static int prologue_passes(int32_t H) {
  const int candidates[3] = {14, 8, 4};
  int best = 14;
  int64_t best_waste = -1;
  for (int p : candidates) {
    const int64_t rows = 4 * p, waste = (2 * (int64_t)H + rows - 1) / rows * rows - 2 * (int64_t)H;
    if (best_waste < 0 || waste < best_waste) best = p, best_waste = waste;
  }
  return best;
}

hipError_t launch_qk_prologue(uint16_t* q, uint16_t* k, const float* gamma_q, const float* gamma_k,
                              const int32_t* pos, int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  const dim3 grid((unsigned)prologue_grid_blocks(L)), block(kWavesPerBlock * 64);
  switch (prologue_passes(H)) {
    case 14:
      hipLaunchKernelGGL(qk_prologue_kernel<14>, grid, block, 0, stream, q, k, gamma_q, gamma_k, pos, L, H, q_scale);
      break;
    case 8:
      hipLaunchKernelGGL(qk_prologue_kernel<8>, grid, block, 0, stream, q, k, gamma_q, gamma_k, pos, L, H, q_scale);
      break;
    default:
      hipLaunchKernelGGL(qk_prologue_kernel<4>, grid, block, 0, stream, q, k, gamma_q, gamma_k, pos, L, H, q_scale);
      break;
  }
  return hipGetLastError();
}

}  // namespace h3attn
