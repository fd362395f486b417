// Full bidirectional (non-causal, unmasked) flash attention forward for gfx950.
//
// Operation ("MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 2 "Attention:
// full bidirectional self-attention"; section 4 "Full attention is non-causal
// and unmasked over one packed document"; section 5 item h3_full_attention):
//   out[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k[j,h,:]>) v[j,h,:]
//
// Numerical contract (same RFC, section 4): fp32 accumulation on the matrix
// cores, one fixed key order (tile 0, 1, 2, ...), no split over keys, no
// atomics; every output row is produced by exactly one wave, so the result
// does not depend on the grid or on the number of CUs.
//
// Work decomposition.  A 256-thread workgroup owns BM = 128 query rows of one
// head; each of its 4 waves owns 32 of them.  The workgroup streams the keys in
// tiles of BN = 64 through LDS (K row-major, V transposed) and every wave runs
//   S^T = K_tile * Q^T        (v_mfma_f32_32x32x16_bf16, 2 x 8 per tile)
//   online softmax on S^T     (fp32; exp2 with scale*log2(e) folded in)
//   O^T += V_tile^T * P^T     (v_mfma_f32_32x32x16_bf16, 4 x 4 per tile)
// Computing the transposed score block makes each lane own one query column
// (lane % 32) and 16 keys of every 32-key block, so the fp32 accumulators of
// S^T convert in place to the bf16 B operand of the P*V product: no LDS round
// trip for P, and the row statistics need one cross-half exchange (lane ^ 32).
// The MFMA k-slot order of P^T is whatever the accumulator layout gives; V^T is
// written to LDS with its key positions permuted to the same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kBM = 128;               // query rows per workgroup
constexpr int kBN = 64;                // keys per tile
constexpr int kThreads = 256;
constexpr int kKPitch = kD + 8;        // bf16 per K row in LDS (272 B: conflict-free 16 B reads)
constexpr int kVPitch = kBN + 8;       // bf16 per V^T row in LDS (144 B)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Key chunk (4 keys) -> LDS position chunk inside each 16-key group.  The
// accumulator of S^T gives lane-half g the keys {4g..4g+3, 8+4g..8+4g+3} of a
// 16-key step; storing key chunks in the order 0, 2, 1, 3 puts exactly those
// 8 keys in LDS positions 8g..8g+7, one 16-byte read.
__device__ __forceinline__ int vt_position(int key_in_tile) {
  const int chunk = (key_in_tile >> 2) & 3;
  const int pchunk = (chunk == 1) ? 2 : (chunk == 2) ? 1 : chunk;
  return (key_in_tile & ~15) | (pchunk << 2) | (key_in_tile & 3);
}

__global__ __launch_bounds__(kThreads) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, int L, int H, float scale_log2e, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBN * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kD * kVPitch];

  // Workgroups are dispatched round-robin over the 8 XCDs (block b -> XCD b%8).
  // Renumber so each XCD receives a contiguous run of (head, q-tile) work:
  // the workgroups that share one head's K/V then share one L2.
  const int nb = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int head = logical / n_qtiles;
  const int qtile = logical - head * n_qtiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int64_t tok_stride = (int64_t)H * kD;  // elements between consecutive tokens
  const int64_t head_off = (int64_t)head * kD;

  // Q^T operand: lane holds Q[row][16ks + 8g .. +7] for its query row.
  const int qrow = qtile * kBM + wave * 32 + col;
  bf16x8_t qf[8];
  if (qrow < L) {
    const uint16_t* p = q + (int64_t)qrow * tok_stride + head_off + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(p + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = bf16x8_t{};
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m_run = -INFINITY;  // running max of raw scores for this lane's query
  float l_run = 0.f;        // this lane-half's partial running sum

  // Cooperative tile loaders.
  // K: 64 keys x 16 sixteen-byte chunks; thread handles chunks tid + 256*it.
  // V: thread handles keys 4*kq..4*kq+3 of d-chunk dc (8 channels); kq varies
  //    fastest across lanes so a wave's transposed LDS writes hit distinct banks.
  const int v_kq = tid & 15, v_dc = tid >> 4;
  const int v_pos = vt_position(4 * v_kq);

  const int n_tiles = (L + kBN - 1) / kBN;
  for (int t = 0; t < n_tiles; ++t) {
    const int kbase = t * kBN;
    __syncthreads();  // all waves are done reading the previous tile
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * kThreads + tid;
      const int key = idx >> 4, dc = idx & 15;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (kbase + key < L)
        val = *reinterpret_cast<const uint4*>(k + (int64_t)(kbase + key) * tok_stride + head_off + 8 * dc);
      *reinterpret_cast<uint4*>(k_lds + key * kKPitch + 8 * dc) = val;
    }
    {
      uint4 vv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int key = kbase + 4 * v_kq + m;
        vv[m] = make_uint4(0u, 0u, 0u, 0u);
        if (key < L)
          vv[m] = *reinterpret_cast<const uint4*>(v + (int64_t)key * tok_stride + head_off + 8 * v_dc);
      }
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vv[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vv[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vv[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vv[3]);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int sh = (d & 1) * 16;
        const uint32_t e0 = (w0[d >> 1] >> sh) & 0xffffu, e1 = (w1[d >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (w2[d >> 1] >> sh) & 0xffffu, e3 = (w3[d >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(vt_lds + (8 * v_dc + d) * kVPitch + v_pos) =
            make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
      }
    }
    __syncthreads();

    // S^T[key][query] for the two 32-key blocks of the tile.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const uint16_t* kr = k_lds + (32 * kb + col) * kKPitch + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8_t*>(kr + 16 * ks), qf[ks], s[kb]);
    }
    // Keys past the end of the document do not exist.
    if (kbase + kBN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            if (kbase + 32 * kb + 8 * r + 4 * g + qq >= L) s[kb][4 * r + qq] = -INFINITY;
    }

    // Online softmax for this lane's query.
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f((m_run - m_new) * scale_log2e);
    const float mc = m_new * scale_log2e;
    float psum = 0.f;
    bf16x8_t pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(fmaf(s[kb][e], scale_log2e, -mc));
        psum += p;
        pf[2 * kb + (e >> 3)][e & 7] = (__bf16)p;
      }
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= alpha;

    // O^T[d][query] += V^T[d][keys] * P^T[keys][query]
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) {
      const uint16_t* vr = vt_lds + (32 * dblk + col) * kVPitch + 8 * g;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        o[dblk] = mfma32(*reinterpret_cast<const bf16x8_t*>(vr + 16 * st), pf[st], o[dblk]);
    }
  }

  // Epilogue: full row sum = both lane-halves; O / l -> bf16.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = 1.0f / l_tot;
  if (qrow < L) {
    uint16_t* po = out + (int64_t)qrow * tok_stride + head_off;
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * dblk + 8 * r + 4 * g;
        *reinterpret_cast<uint2*>(po + d) =
            make_uint2(pack_bf16x2(o[dblk][4 * r] * inv_l, o[dblk][4 * r + 1] * inv_l),
                       pack_bf16x2(o[dblk][4 * r + 2] * inv_l, o[dblk][4 * r + 3] * inv_l));
      }
  }
}

}  // namespace

int64_t attention_grid_blocks(int64_t L, int32_t H) { return ((L + kBM - 1) / kBM) * (int64_t)H; }

hipError_t launch_attention_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, int64_t L, int32_t H, float scale,
                                    hipStream_t stream) {
  const int n_qtiles = (int)((L + kBM - 1) / kBM);
  const dim3 grid((unsigned)attention_grid_blocks(L, H));
  hipLaunchKernelGGL(attention_fwd_kernel, grid, dim3(kThreads), 0, stream, q, k, v, out, (int)L,
                     (int)H, scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

}  // namespace h3attn
