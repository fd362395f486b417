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
// head; each of its 4 waves owns 32 of them.  Keys stream through LDS in tiles
// of BN = 64, double-buffered: while the waves compute on tile t, the DMA
// loads of tile t+1 (global_load_lds_dwordx4, no VGPR staging) fill the other
// buffer; one barrier per tile.  Per tile every wave runs
//   S^T = K_tile * Q^T        (v_mfma_f32_32x32x16_bf16, 2 x 8)
//   online softmax on S^T     (fp32; exp2 with scale*log2(e) folded into an FMA)
//   O^T += V_tile^T * P^T     (v_mfma_f32_32x32x16_bf16, 4 x 4)
// Computing the transposed score block makes each lane own one query column
// (lane % 32) and 16 keys of every 32-key block, so the fp32 accumulators of
// S^T convert in place to the bf16 B operand of the P*V product (no LDS round
// trip for P), and the row statistics need one cross-half exchange (lane ^ 32).
//
// LDS layout.  K and V tiles are both stored row-major (one 256-byte row per
// key, sixteen 16-byte chunks) with chunk c of row r at physical chunk
// c ^ swz(r), swz(r) = 4*(r & 3) + ((r >> 2) & 3).  The LDS has 64 four-byte
// banks (one 256-byte row) and serves 16 lanes of a 16-byte read, or 32 lanes
// of an 8-byte read, per cycle.  swz takes 16 distinct values over any 16
// consecutive rows, so the K operand read (16 rows, one chunk) is
// conflict-free; and for 4 consecutive rows its top two bits are distinct, so
// the transposed V read (ds_read_b64_tr_b16: 32 lanes = 4 consecutive keys x
// 4 aligned chunks; each lane receives 4 consecutive keys of one channel) is
// conflict-free too.  Both were checked with the SQ_LDS_BANK_CONFLICT counter.
//
// Softmax rescaling is lazy: the running maximum m used as the exponent offset
// only moves when a tile's maximum exceeds it by more than 8 (in log2 units), so
// P <= 2^8 and the O rescale is skipped on almost every tile.  The final O / l
// is unchanged by the choice of offset because l sums exactly the bf16 P values
// that enter the P*V product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;

constexpr int kD = 128;
constexpr int kBM = 128;                 // query rows per workgroup
constexpr int kBN = 64;                  // keys per tile
constexpr int kThreads = 256;
constexpr int kTileBytes = kBN * kD * 2; // 16 KiB per K or V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Byte offset of (row, channel) in a swizzled tile; channel % 4 == 0.
__device__ __forceinline__ int tile_offset(int row, int ch) {
  return row * (kD * 2) + ((((ch >> 3) ^ swz(row))) << 4) + ((ch & 7) << 1);
}

// DMA one 64-key tile of a [L][H][128] tensor into a swizzled LDS tile.  Each
// wave writes four contiguous 1 KiB pieces (64 lanes x 16 B, lane-ordered);
// lane `lane` of piece p fetches the global chunk that belongs at its slot.
// The tile base is wave-uniform and each lane adds a fixed 32-bit byte offset
// (row * token stride + chunk), so per tile only the scalar base moves.
struct DmaOffsets {
  uint32_t off[4];
};

__device__ __forceinline__ DmaOffsets dma_offsets(int64_t tok_stride, int wave, int lane, int max_row) {
  DmaOffsets d;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int slot = (it * 4 + wave) * 64 + lane;  // 16-byte slot in the tile
    const int r = slot >> 4;
    const int c = (slot & 15) ^ swz(r);
    // Rows past the end of the document re-read the last row (finite values;
    // their scores are masked and their probabilities are zero).
    d.off[it] = (uint32_t)(((int64_t)min(r, max_row) * tok_stride + 8 * c) * 2);
  }
  return d;
}

__device__ __forceinline__ void tile_dma(const char* tile_base, const DmaOffsets& d, lds_char* tile,
                                         int wave) {
#pragma unroll
  for (int it = 0; it < 4; ++it)
    __builtin_amdgcn_global_load_lds(tile_base + d.off[it], tile + (it * 4 + wave) * 1024, 16, 0, 0);
}

// One tile: S^T, online softmax, O^T += V^T P^T.  kt/vt are the tile's LDS buffers.
template <bool kTail>
__device__ __forceinline__ void tile_step(const lds_char* kt, const lds_char* vt, const bf16x8_t (&qf)[8],
                                          f32x16_t (&o)[4], float& m_run, float& l_run, int kbase,
                                          int L, float c, int col, int g, int lane) {
  // S^T[key][query] for the two 32-key blocks of the tile; the two accumulation
  // chains are interleaved so consecutive MFMAs are independent.
  f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8_t a = *(const lds_bf16x8*)(kt + tile_offset(32 * kb + col, 16 * ks + 8 * g));
      s[kb] = mfma32(a, qf[ks], s[kb]);
    }
  }
  if (kTail) {  // keys past the end of the document do not exist
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (kbase + 32 * kb + 8 * r + 4 * g + qq >= L) s[kb][4 * r + qq] = -INFINITY;
  }

  // Tile maximum of this lane's query over both lane-halves.
  float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(s[0][e], s[1][e]));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // Move the exponent offset only when the tile would push P above 2^8.  Both
  // lane-halves of a query see the same mx and m_run, so they decide alike.
  const bool need = (mx - m_run) * c > kRescaleThreshold;
  if (__any(need)) {
    const float m_new = need ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);  // m_run = -inf on the first tile -> 0
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= alpha;
    m_run = m_new;
  }
  // P = 2^(s*c - m*c), rounded to bf16 for the P*V product.  The row sum adds
  // the same rounded values (v_dot2_f32_bf16 against (1, 1)), so the output is
  // an exact convex combination of V rows with the weights the MFMA used.
  const float mc = m_run * c;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8_t pf[4];
  float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      bf16x2_t pr;
      pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][e], c, -mc));
      pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][e + 1], c, -mc));
      psum[e >> 2 & 3] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psum[e >> 2 & 3], false);
      pf[2 * kb + (e >> 3)][e & 7] = pr[0];
      pf[2 * kb + (e >> 3)][(e & 7) + 1] = pr[1];
    }
  l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);

  // O^T[d][query] += V^T[d][keys] * P^T[keys][query].  The A operand for d-block
  // dblk and 16-key step st comes from two transposed reads: lane l (group
  // G = l >> 4, index i = l & 15) addresses key 16*st + 4*(G >> 1) + (i >> 2)
  // (+8 for the second read) at channel 32*dblk + 16*(G & 1) + 4*(i & 3), and
  // receives keys {16 st + 4g + e} and {16 st + 8 + 4g + e} of channel
  // 32*dblk + (l % 32) -- the same key order as the P^T accumulator slots.
  const int G = lane >> 4, i = lane & 15;
  const int key_a = 4 * (G >> 1) + (i >> 2);
  const int ch = 16 * (G & 1) + 4 * (i & 3);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) {
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vt + tile_offset(16 * st + key_a, 32 * dblk + ch)));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vt + tile_offset(16 * st + 8 + key_a, 32 * dblk + ch)));
      typedef short i16x8_t __attribute__((ext_vector_type(8)));
      const i16x8_t a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dblk] = mfma32(__builtin_bit_cast(bf16x8_t, a16), pf[st], o[dblk]);
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, int L, int H, float scale_log2e, int n_qtiles) {
  __shared__ __attribute__((aligned(1024))) char k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[kTileBytes];

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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int64_t tok_stride = (int64_t)H * kD;  // elements between consecutive tokens
  const uint16_t* kh = k + (int64_t)head * kD;
  const uint16_t* vh = v + (int64_t)head * kD;

  const int n_full = L / kBN;                 // tiles with 64 real keys
  const int n_tiles = (L + kBN - 1) / kBN;    // plus one partial tile if L % 64 != 0
  const int64_t tile_stride_bytes = (int64_t)kBN * tok_stride * 2;
  const char* kbase_ptr = reinterpret_cast<const char*>(kh);
  const char* vbase_ptr = reinterpret_cast<const char*>(vh);
  const DmaOffsets dma_full = dma_offsets(tok_stride, wave, lane, kBN - 1);
  const DmaOffsets dma_tail = dma_offsets(tok_stride, wave, lane, (L - 1) % kBN);
  auto dma = [&](int t, lds_char* kt, lds_char* vt) {
    const DmaOffsets& d = (t < n_full) ? dma_full : dma_tail;
    tile_dma(kbase_ptr + t * tile_stride_bytes, d, kt, wave);
    tile_dma(vbase_ptr + t * tile_stride_bytes, d, vt, wave);
  };
  dma(0, (lds_char*)k_lds0, (lds_char*)v_lds0);

  // Q^T operand: lane holds Q[row][16ks + 8g .. +7] for its query row.
  const int qrow = qtile * kBM + wave * 32 + col;
  bf16x8_t qf[8];
  if (qrow < L) {
    const uint16_t* p = q + (int64_t)qrow * tok_stride + (int64_t)head * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(p + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = bf16x8_t{};
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m_run = -INFINITY;  // exponent offset (raw score units) for this lane's query
  float l_run = 0.f;        // this lane-half's partial sum of P
  auto full_step = [&](int t, const lds_char* kt, const lds_char* vt) {
    tile_step<false>(kt, vt, qf, o, m_run, l_run, t * kBN, L, scale_log2e, col, g, lane);
  };
  __syncthreads();          // tile 0 is in LDS

  // Full tiles, two per trip so each buffer is named statically; the loop body
  // is one straight path.  The partial tile (if L % 64 != 0) is peeled below.
  int t = 0;
  for (; t + 1 < n_full; t += 2) {
    dma(t + 1, (lds_char*)k_lds1, (lds_char*)v_lds1);
    full_step(t, (const lds_char*)k_lds0, (const lds_char*)v_lds0);
    __syncthreads();  // tile t+1 landed; every wave is done with buffer 0
    if (t + 2 < n_tiles) dma(t + 2, (lds_char*)k_lds0, (lds_char*)v_lds0);
    full_step(t + 1, (const lds_char*)k_lds1, (const lds_char*)v_lds1);
    __syncthreads();  // tile t+2 landed; every wave is done with buffer 1
  }
  if (t < n_full) {  // odd number of full tiles: the last one sits in buffer 0
    if (t + 1 < n_tiles) dma(t + 1, (lds_char*)k_lds1, (lds_char*)v_lds1);
    full_step(t, (const lds_char*)k_lds0, (const lds_char*)v_lds0);
    __syncthreads();
    ++t;
  }
  if (t < n_tiles) {  // the partial tile, in buffer t % 2
    const lds_char* kt = (t & 1) ? (const lds_char*)k_lds1 : (const lds_char*)k_lds0;
    const lds_char* vt = (t & 1) ? (const lds_char*)v_lds1 : (const lds_char*)v_lds0;
    tile_step<true>(kt, vt, qf, o, m_run, l_run, t * kBN, L, scale_log2e, col, g, lane);
  }

  // Epilogue: full row sum = both lane-halves; O / l -> bf16.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = 1.0f / l_tot;
  if (qrow < L) {
    uint16_t* po = out + (int64_t)qrow * tok_stride + (int64_t)head * kD;
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
