// Backward of full bidirectional (non-causal, unmasked) attention for gfx950.
//
// Why: the "MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 7 ("Acceptance
// gates", per-operator gate) asks for forward and backward of each operator;
// the operator is its section 5 work item h3_full_attention.
//
// Operation, per head, with S = scale Q K^T (Q, K the prologue outputs),
// P = softmax rows of S, O = P V, and dO the gradient of the output:
//   dV = P^T dO
//   dP = dO V^T,  delta_i = sum_d dO_id O_id,  dS = P * (dP - delta)
//   dQ = scale dS K,  dK = scale dS^T Q
// P is recomputed from the forward's log-sum-exp: P_ij = 2^(c s_ij - lse_i log2 e),
// c = scale log2 e, with keys and queries past L excluded.
//
// Numerical contract as in the forward: bf16 operands on the matrix cores
// (P and dS are rounded to bf16 where they become an operand), fp32
// accumulation, one fixed order over the streamed rows, no atomics and no
// split: every output row is produced by exactly one wave, so results do not
// depend on the grid.
//
// Two kernels; each wave owns 32 rows of one head and the workgroup streams
// the other side through LDS in 64-row tiles:
//   dq (8 waves, 256 queries): streams K and V.  Per 32-key block S^T = K Q^T
//        and dP^T = V dO^T (K, V row operands from LDS; Q^T, dO^T held in
//        registers), dS^T from them, dQ^T += K^T dS^T (K^T gathered by
//        transposing LDS reads), software-pipelined over the blocks.  It
//        also computes delta for its rows and leaves -lse log2(e) and -delta
//        per row for the second kernel.
//   dkdv (4 waves, 128 keys): streams Q, dO and those two statistics.  Per
//        32-query block S = Q K^T and dP - delta = dO V^T - delta (Q, dO from
//        LDS; K^T, V^T in registers), P and dS, dV^T += dO^T P and
//        dK^T += Q^T dS, software-pipelined over the blocks.
// Computing the transposed product of the side whose rows the wave owns puts
// one of its rows in each lane column, so the fp32 accumulators of S (or
// S^T) convert in place to the bf16 B operand of the next product, in the
// key (query) order that the transposing reads of the streamed tile produce
// -- the same layout the forward kernel uses for P^T V.  The dkdv kernel keeps
// both accumulator sets and both operand sets: one wave per SIMD gives it 512
// registers (at two waves per SIMD the fused kernel spills; split into a dK
// and a dV kernel it recomputes S once more and takes 11% longer).
//
// Tiles arrive by buffer_load_dwordx4 ... lds into a ring of four slots (no
// VGPR staging), one barrier per tile; tiles are row-major with chunk c of
// row r at c ^ swz(r) (conflict-free row and transposing reads).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gfx950_tile.h"
#include "h3attn_internal.h"

namespace h3attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;                       // rows a workgroup owns
constexpr int kTile = 64;                                // rows per streamed tile
constexpr int kTileBytes = kTile * kD * 2;               // 16 KiB
constexpr float kLog2e = 1.4426950408889634f;
// ---------------------------------------------------------------- tile DMA
// A 64-row tile of a [L][H][128] tensor: 16 pieces of 1 KiB, wave w writing
// pieces w and w + 8; slot (row r, physical chunk p) <- row r, channels
// 8 (p ^ swz(r)) .. +7.  The buffer resource ends at the tensor's last row,
// so rows past L read as zeros and no address leaves the tensor.
template <int W>
constexpr int dma_per_wave() { return kTileBytes / 1024 / W; }  // pieces per wave per tile

template <int W>
struct DmaOffsets {
  uint32_t off[dma_per_wave<W>()];
};

template <int W>
__device__ __forceinline__ DmaOffsets<W> dma_offsets(int64_t tok_stride, int wave, int lane) {
  DmaOffsets<W> d;
#pragma unroll
  for (int it = 0; it < dma_per_wave<W>(); ++it) {
    const int slot = (it * W + wave) * 64 + lane;
    const int r = slot >> 4;
    const int c = (slot & 15) ^ swz(r);
    d.off[it] = (uint32_t)(((int64_t)r * tok_stride + 8 * c) * 2);
  }
  return d;
}

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, int64_t valid_bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t n = valid_bytes <= 0 ? 0u : valid_bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)valid_bytes;
  return i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
                 (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)),
                 (int)__builtin_amdgcn_readfirstlane(n), kBufferDword3};
}

// Piece it of this wave's share of row tile t of the tensor at base (this
// head's row 0; rows tok_stride elements apart) into LDS at lds_tile (W waves
// share a tile, dma_per_wave<W>() pieces each).
template <int W>
__device__ __forceinline__ void dma_row_piece(const uint16_t* base, int64_t tok_stride, int t, int L,
                                              const DmaOffsets<W>& d, uint32_t lds_tile, int wave, int it) {
  const int64_t row_bytes = tok_stride * 2;
  const i32x4_t rsrc = buffer_rsrc(base + (int64_t)t * kTile * tok_stride,
                                   (int64_t)(L - 1 - t * kTile) * row_bytes + kD * 2);
  lds_dma_dwordx4(rsrc, d.off[it], __builtin_amdgcn_readfirstlane(lds_tile + (it * W + wave) * 1024));
}

// The 64 fp32 values v[t*64 .. t*64+63] of an n-value vector (zeros past n)
// into LDS at lds: one 1 KiB piece, whose first 256 bytes are those values.
__device__ __forceinline__ void dma_vec(const float* v, int t, int n, uint32_t lds, int lane) {
  lds_dma_dwordx4(buffer_rsrc(v + (int64_t)t * kTile, (int64_t)(n - t * kTile) * 4), 16u * lane,
                  __builtin_amdgcn_readfirstlane(lds));
}

// ---------------------------------------------------------------- LDS operands
// Row operand of a tile (32-row block blk, k-step ks): lane reads row
// 32 blk + col, channels 16 ks + 8 g .. +7 (the A operand whose rows are the
// tile's rows).  Transposing operand (d-block dblk, 16-row step j): lane
// receives channel 32 dblk + col of rows 16 j + {4g .. 4g+3, 8+4g .. 11+4g},
// by two ds_read_b64_tr_b16 -- the row order of a 32x32 accumulator's slots
// in lane half g, so a packed accumulator is the matching B operand.
struct Addr {
  uint32_t row, tr0, tr1;
};

__device__ __forceinline__ Addr lds_addresses(int lane) {
  const int col = lane & 31, g = lane >> 5;
  const int key_a = 4 * g + ((lane & 15) >> 2);             // transposing-read row of this lane
  const int ch = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);    // transposing-read channel
  Addr a;
  a.row = 256u * col + ((16u * g) ^ (16u * swz(col)));
  a.tr0 = 256u * key_a + 8u * ((ch >> 2) & 1) + ((16u * (ch >> 3)) ^ (16u * swz(key_a)));
  a.tr1 = 256u * (8 + key_a) + 8u * ((ch >> 2) & 1) + ((16u * (ch >> 3)) ^ (16u * swz(8 + key_a)));
  return a;
}

__device__ __forceinline__ bf16x8_t row_operand(const lds_char* tile, int blk, int ks, const Addr& a) {
  return *(const lds_bf16x8*)(tile + blk * 8192 + (a.row ^ (32u * ks)));
}

__device__ __forceinline__ bf16x8_t tr_operand(const lds_char* tile, int dblk, int j, const Addr& a) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + 4096 * j + (a.tr0 ^ (64u * dblk))));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + 4096 * j + (a.tr1 ^ (64u * dblk))));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 32-row block of a [L][H][128] tensor as the B operand of a 32x32x16
// MFMA: lane holds row (row0 + col), channels 16 ks + 8 g .. +7; zeros past L.
__device__ __forceinline__ void load_row_operands(const uint16_t* base, int64_t tok_stride, int row, int L, int g,
                                                  bf16x8_t (&op)[8]) {
  if (row < L) {
    const uint16_t* p = base + (int64_t)row * tok_stride + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) op[ks] = *reinterpret_cast<const bf16x8_t*>(p + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) op[ks] = bf16x8_t{};
  }
}

// acc[dblk][4 rr + qq] = X^T[32 dblk + 8 rr + 4 g + qq][col] -> x[row][d] * f, bf16.
__device__ __forceinline__ void store_transposed(uint16_t* row_ptr, const f32x16_t (&acc)[4], float f, int g) {
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = 32 * dblk + 8 * rr + 4 * g;
      *reinterpret_cast<uint2*>(row_ptr + d) =
          make_uint2(pack_bf16x2(acc[dblk][4 * rr] * f, acc[dblk][4 * rr + 1] * f),
                     pack_bf16x2(acc[dblk][4 * rr + 2] * f, acc[dblk][4 * rr + 3] * f));
    }
}

// Blocks b < H * n_full take the full 256-row tiles, renumbered so each XCD
// (block b -> XCD b % 8) gets a contiguous run of them; the last H blocks
// take each head's partial tile.
__device__ __forceinline__ void block_tile(int b, int H, int n_full, int& head, int& tile) {
  const int nfb = H * n_full;
  if (b < nfb) {
    const int xcd = b & 7, slot = b >> 3, per = nfb >> 3, rem = nfb & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    head = logical / n_full;
    tile = logical - head * n_full;
  } else {
    head = b - nfb;
    tile = n_full;
  }
}

// The dq kernel's blocks: as block_tile, except that the last n_half full
// 256-row tiles (in head-major order) run as two workgroups of 128 rows each
// (blocks H n_full - n_half .. H n_full + n_half - 1), whose waves 0..3 own
// the rows; those workgroups finish sooner and fill a last round that would
// otherwise leave CUs idle.  active: the waves that own rows.
__device__ __forceinline__ void dq_tile(int b, int H, int n_full, int n_half, int& head, int& row0, int& active) {
  const int nfb = H * n_full;
  active = kWaves;
  if (b < nfb - n_half) {
    const int nwhole = nfb - n_half, xcd = b & 7, slot = b >> 3, per = nwhole >> 3, rem = nwhole & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    head = logical / n_full;
    row0 = (logical - head * n_full) * kRows;
  } else if (b < nfb + n_half) {
    const int j = b - (nfb - n_half), logical = nfb - n_half + (j >> 1);
    head = logical / n_full;
    row0 = (logical - head * n_full) * kRows + (j & 1) * (kRows / 2);
    active = kWaves / 2;
  } else {
    head = b - nfb - n_half;
    row0 = n_full * kRows;
  }
}

// ---------------------------------------------------------------- dq (+ delta)
// Software-pipelined over 32-key blocks, like the dk/dv kernel below but at
// two waves per SIMD: block (t, kb) is the kb-th half of key tile t, and the
// step of a block issues, over 24 matrix slots,
//   S^T = K Q^T and dP^T = V dO^T of the next block   (16 MFMAs)
//   dQ^T += K^T dS^T of the previous block            (8 MFMAs)
// and this block's weights, P = exp2(c S - lse log2 e), dS = P (dP - delta).
// Slot k with k % 3 == 2 holds dQ MFMA k / 3 (= 4 jj + dblk); every other
// slot holds MFMA n = 2 (k / 3) + k % 3 of the next block, S for even n and dP
// for odd n, k-step n / 2.  Element e of this block's weights starts at slot
// e (exponent), then its exponential, then dS, and each bf16 pair is packed
// the slot after its second dS; the last slots hold matrix work only (this
// front-loaded order measured 1% faster than one spread over all 24 slots).
// K and V come through rings of four 64-key tiles (128 KiB); the step of
// (t, 0) starts the DMA of tile t + 2 into the slot of tile t - 2 and ends
// with the tile's one barrier.
//
// The dP^T chain starts from -delta instead of 0, so it leaves the matrix
// core as dP - delta and dS is one multiplication; when c = scale log2(e) is
// exactly 1 (the scale-folded layout's scale ln 2), the S^T chain likewise
// starts from -lse log2(e) - 1, and the weight is one exponential with no FMA
// in front of it.  Both starts are one value per lane (its query row),
// written into the accumulators at the top of each step.
//
// The weights are computed halved, P/2 = exp2(c S - lse log2 e - 1) with the
// exponential's output clamped to [0, 1] (a free instruction modifier), and dQ
// is scaled by 2 scale at the end: every true weight is at most 1 (up to the
// forward's rounding of lse), so the clamp never touches one, while keys past
// L (in the last tile only), whose K and V rows read as zeros, get a finite
// weight whatever the row's log-sum-exp -- their dS then adds K-row zeros to
// dQ with no test.
constexpr int kDqStages = 4;
constexpr int kDqPieces = 2 * dma_per_wave<kWaves>();  // K and V pieces per wave per tile

__device__ __forceinline__ bf16x8_t dq_operand(int k, const lds_char* nk, const lds_char* nv, int kbn,
                                               const lds_char* pk, int kbp, const Addr& a) {
  if (k % 3 == 2) {
    const int i = k / 3;
    return tr_operand(pk, i & 3, 2 * kbp + (i >> 2), a);
  }
  const int n = 2 * (k / 3) + k % 3;
  return row_operand((n & 1) ? nv : nk, kbn, n >> 1, a);
}

constexpr int dq_slot(int e) { return e; }
// Slots a step runs: the 24 matrix slots, and after them any the last pair's pack needs.
constexpr int kDqSteps = dq_slot(15) + 4 > 24 ? dq_slot(15) + 4 : 24;

// One step: next block in K/V slots nk, nv (half kbn), previous block in K
// slot pk (half kbp; kPrev: there is one).  s_c, dp_c: this block's S^T and
// dP^T; s_n, dp_n: the next block's; ds_p: the previous block's dS^T / 2
// operand, ds_c: this block's.  nl = -lse log2(e) - 1, dl = delta of the
// lane's query row; kUnit: c == 1, the S^T chain starts from nl.
template <bool kPrev, bool kUnit, typename Dma>
__device__ __forceinline__ void dq_step(const lds_char* nk, const lds_char* nv, int kbn, const lds_char* pk, int kbp,
                                        const Addr& a, float c, float nl, float dl, const f32x16_t& s_c,
                                        const f32x16_t& dp_c, f32x16_t& s_n, f32x16_t& dp_n,
                                        const bf16x8_t (&ds_p)[2], bf16x8_t (&ds_c)[2], f32x16_t (&acc)[4],
                                        const bf16x8_t (&qop)[8], const bf16x8_t (&dop)[8], const Dma& dma) {
  constexpr int kAheadDq = 2;
  // The chains' start values, made opaque here so that the compiler builds
  // them in the accumulators each step instead of holding a broadcast copy of
  // each (32 registers) through the loop.
  float nls = nl, ndl = -dl;
  asm volatile("" : "+v"(nls), "+v"(ndl));
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    s_n[e] = kUnit ? nls : 0.f;
    dp_n[e] = ndl;
  }
  bf16x8_t op[24];
#pragma unroll
  for (int j = 0; j < kAheadDq; ++j)
    if (kPrev || j % 3 != 2) op[j] = dq_operand(j, nk, nv, kbn, pk, kbp, a);
  __builtin_amdgcn_sched_barrier(0);
  float xa[16], p[16], x[16];
  uint32_t pair[8];
#pragma unroll
  for (int k = 0; k < kDqSteps; ++k) {
    dma(k);
    if (k < 24) {
      const int kk = k + kAheadDq;
      if (kk < 24 && (kPrev || kk % 3 != 2)) op[kk] = dq_operand(kk, nk, nv, kbn, pk, kbp, a);
      if (k % 3 == 2) {
        if (kPrev) {
          const int i = k / 3;
          acc[i & 3] = mfma32(op[k], ds_p[i >> 2], acc[i & 3]);
        }
      } else {
        const int n = 2 * (k / 3) + k % 3;
        if (n & 1) dp_n = mfma32(op[k], dop[n >> 1], dp_n);
        else s_n = mfma32(op[k], qop[n >> 1], s_n);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (k == dq_slot(e)) xa[e] = kUnit ? s_c[e] : fmaf(s_c[e], c, nl);
      if (k == dq_slot(e) + 1) p[e] = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(xa[e]), 0.f, 1.f);
      if (k == dq_slot(e) + 2) x[e] = p[e] * dp_c[e];
    }
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (k == dq_slot(2 * m + 1) + 3) pair[m] = pack_bf16x2(x[2 * m], x[2 * m + 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
    ds_c[h] = __builtin_bit_cast(bf16x8_t, u32x4_t{pair[4 * h], pair[4 * h + 1], pair[4 * h + 2], pair[4 * h + 3]});
}

template <bool kUnit>
__global__ __launch_bounds__(kThreads, 1) void attention_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ out, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    uint16_t* __restrict__ dq, float* __restrict__ stats, int L, int H, int Lp, float c, float scale, int n_full,
    int n_half) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kDqStages * kTileBytes];  // K ring, then V ring
  int head, row0, active;
  dq_tile(blockIdx.x, H, n_full, n_half, head, row0, active);
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tok_stride = (int64_t)H * kD;
  const int n_tiles = (L + kTile - 1) / kTile;
  const lds_char* lds = (const lds_char*)lds_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)lds_raw;
  const DmaOffsets<kWaves> dmo = dma_offsets<kWaves>(tok_stride, wave, lane);
  const uint16_t* kh = k + (int64_t)head * kD;
  const uint16_t* vh = v + (int64_t)head * kD;
  // DMA piece j of tile t (clamped to the last tile: refetches keep the count
  // per step fixed): the first half K, the second V.
  constexpr int kHalf = kDqPieces / 2;
  auto piece = [&](int t, int j) {
    const int tt = t < n_tiles ? t : n_tiles - 1;
    const uint32_t s = lds_base + (uint32_t)(t % kDqStages) * kTileBytes;
    if (j < kHalf) dma_row_piece<kWaves>(kh, tok_stride, tt, L, dmo, s, wave, j);
    else dma_row_piece<kWaves>(vh, tok_stride, tt, L, dmo, s + kDqStages * kTileBytes, wave, j - kHalf);
  };
  const auto kslot = [&](int t) { return lds + (t % kDqStages) * kTileBytes; };
  const auto vslot = [&](int t) { return lds + (kDqStages + t % kDqStages) * kTileBytes; };
  constexpr int kEvery = 24 / kDqPieces;  // the step issues one piece every kEvery slots
  static_assert(kEvery * kDqPieces == 24, "the pieces spread evenly over the 24 slots");
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) piece(t, j);

  const bool owner = wave < active;  // this wave's rows belong to this workgroup
  const int row = row0 + wave * 32 + col;
  const bool valid = owner && row < L;
  const int lrow = owner ? row : L;  // rows past L load as zeros
  bf16x8_t qop[8], dop[8];
  load_row_operands(q + (int64_t)head * kD, tok_stride, lrow, L, g, qop);
  load_row_operands(dout + (int64_t)head * kD, tok_stride, lrow, L, g, dop);
  float dsum = 0.f;  // delta = <dO, O> over this lane's 64 channels, then both halves
  {
    bf16x8_t oop[8];
    load_row_operands(out + (int64_t)head * kD, tok_stride, lrow, L, g, oop);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) dsum = fmaf((float)dop[ks][i], (float)oop[ks][i], dsum);
  }
  const float dl = pair_sum(dsum);
  const float lse2 = valid ? lse[(int64_t)head * L + row] * kLog2e : 0.f;
  if (owner && g == 0 && row < Lp) {  // statistics for the dk/dv kernel; rows L .. Lp-1 get weight 0 there
    stats[(int64_t)head * Lp + row] = valid ? -lse2 : -INFINITY;
    stats[((int64_t)H + head) * Lp + row] = valid ? -dl : 0.f;
  }
  const float nl = -lse2 - 1.0f;  // halved weights (see above)
  const Addr a = lds_addresses(lane);

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
  dma_wait();
  __syncthreads();

  // A wave none of whose rows exists (in a head's last, partial query tile)
  // or that owns none (waves 4..7 of a half tile) carries its share of the
  // ring DMA and takes part in every barrier, computing nothing: its SIMD's
  // matrix core is left to the other wave.
  if (!owner || row0 + wave * 32 >= L) {
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) piece(2, j);
    dma_wait_all_but<kDqPieces>();
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
#pragma unroll
      for (int j = 0; j < kDqPieces; ++j) piece(t + 3, j);
      dma_wait_all_but<kDqPieces>();
      __syncthreads();
    }
    dma_wait();
    return;
  }

  // Block (0, 0)'s scores.
  f32x16_t sa, da;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    sa[e] = kUnit ? nl : 0.f;
    da[e] = -dl;
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    sa = mfma32(row_operand(kslot(0), 0, ks, a), qop[ks], sa);
    da = mfma32(row_operand(vslot(0), 0, ks, a), dop[ks], da);
  }
  // The last trip's second step, block (n_tiles, 0), finishes dQ of the last
  // block; its own scores come from a stale (loaded) slot and are never used.
  f32x16_t sb, db;
  bf16x8_t dsa[2], dsb[2];
  const auto no_dma = [](int) {};
  {
    const auto dma = [&](int ks) {
      if (ks % kEvery == 1 && ks < 24) piece(2, ks / kEvery);
    };
    dq_step<false, kUnit>(kslot(0), vslot(0), 1, kslot(0), 0, a, c, nl, dl, sa, da, sb, db, dsb, dsa, acc, qop, dop, dma);
    dma_wait_all_but<kDqPieces>();  // tile 1 landed; tile 2 may be in flight
    __syncthreads();
  }
  for (int t = 0; t < n_tiles; ++t) {
    dq_step<true, kUnit>(kslot(t + 1), vslot(t + 1), 0, kslot(t), 0, a, c, nl, dl, sb, db, sa, da, dsa, dsb, acc, qop, dop,
                  no_dma);
    const auto dma = [&](int ks) {
      if (ks % kEvery == 1 && ks < 24) piece(t + 3, ks / kEvery);
    };
    dq_step<true, kUnit>(kslot(t + 1), vslot(t + 1), 1, kslot(t), 1, a, c, nl, dl, sa, da, sb, db, dsb, dsa, acc, qop, dop,
                  dma);
    dma_wait_all_but<kDqPieces>();
    __syncthreads();
  }
  dma_wait();
  // The row's 64-bit offset again (an opaque copy of row keeps the compiler
  // from holding the one computed for the loads through the loop).
  int orow = row;
  asm volatile("" : "+v"(orow));
  if (valid) store_transposed(dq + (int64_t)orow * tok_stride + (int64_t)head * kD, acc, 2.0f * scale, g);
}

// ---------------------------------------------------------------- dk, dv
// Statistics from the dq kernel (the workspace), fp32 [2][H][Lp]: -lse_i
// log2(e), then -delta_i, with -inf and 0 in rows L .. Lp-1 so that a query
// row past L gets weight exp2(-inf) = 0 without a test.
//
// Ring slot: Q tile, dO tile, then one 1 KiB DMA piece per statistic (the
// tile's 64 values in its first 256 bytes).
constexpr int kSlotBytes = 2 * kTileBytes + 2048;
constexpr int kFusedStages = 4;
constexpr int kFusedWaves = 4;
constexpr int kFusedRows = 32 * kFusedWaves;
constexpr int kFusedPieces = 2 * dma_per_wave<kFusedWaves>();  // Q and dO pieces per wave per tile
constexpr int kAhead = 4;                                       // operand reads this many slots early

// dK and dV in one pass over the queries (S computed once per tile): a
// workgroup of 4 waves, one per SIMD, owning 128 keys.  One wave per SIMD has
// 512 registers: the two accumulator sets and the scores and weights of two
// blocks in VGPRs, the K^T, V^T operands (read only by the matrix cores) in
// AGPRs; the build keeps matrix accumulators in VGPRs, so the vector units
// read the scores where the matrix cores leave them.
//
// With no second wave on the SIMD to fill the matrix cores while the vector
// units compute weights, the wave does it itself: the queries are taken in
// 32-row blocks, and the step of block b issues, slot by slot,
//   S(b+1) = Q K^T, dP'(b+1) = dO V^T - delta   (16 MFMAs; the dP' chain starts
//                                                 from -delta instead of 0)
//   dV^T += dO(b-1)^T P(b-1), dK^T += Q(b-1)^T dS(b-1)   (16 MFMAs)
//   P(b) = exp2(c S - lse log2 e), dS(b) = P dP'  (vector units)
// none of which depends on another.  Block (t, h) is the h-th half of query
// tile t.  The step of (t, 0) also starts the DMA of tile t + 2 into the slot
// of tile t - 2 (last read by the step of (t - 1, 0)), and ends with the one
// barrier of the tile, after which tile t + 1 (read from the step of (t, 1)
// on) has landed: each DMA has three steps to arrive.
struct FusedOps {
  f32x16_t dka[4], dva[4];
  bf16x8_t kop[8], vop[8];
};

// LDS operand of matrix slot k of a step: even k, MFMA k/2 of the next block's
// S (k/2 even) or dP' (odd), k-step k/4, from its Q or dO rows; odd k, MFMA
// i = (k-1)/2 = 8 jj + 2 dblk + w of the previous block's dV (w = 0, from dO)
// or dK (w = 1, from Q), 16-row step 2 qbp + jj, by transposing reads.
__device__ __forceinline__ bf16x8_t fused_operand(int k, const lds_char* nxt, int qbn, const lds_char* prv,
                                                  int qbp, const Addr& a) {
  const int i = k >> 1;
  if ((k & 1) == 0) return row_operand(nxt + (i & 1) * kTileBytes, qbn, i >> 1, a);
  return tr_operand(prv + ((i & 1) ? 0 : kTileBytes), (i >> 1) & 3, 2 * qbp + (i >> 3), a);
}

// The step of one block (slot cur, half qb): next block in slot nxt, half qbn;
// previous block in slot prv, half qbp (kPrev: there is one).  s_c, dp_c: this
// block's S and dP'; s_n, dp_n: the next block's, computed here; w*_p: the
// previous block's packed P and dS (B operands), w*_c: this block's.  Slot k
// of this block's weights: 2e the exponent of score e, 2e+1 its exponential,
// 2e+2 dS = P dP', and each bf16 pair packed the slot after its second value;
// dma(k) issues the step's share of the ring DMA.
//
// kUnit (c == 1, the scale-folded layout's scale ln 2): the S chain of the
// next block starts from its rows' -lse log2(e) instead of 0, as the dP' chain
// starts from -delta, so a score leaves the matrix core as its exponent and
// the weight is one exponential with no FMA in front of it.
template <bool kPrev, bool kUnit, typename Dma>
__device__ __forceinline__ void fused_step(const lds_char* cur, int qb, const lds_char* nxt, int qbn,
                                           const lds_char* prv, int qbp, const Addr& a, float c, int g,
                                           const f32x16_t& s_c, const f32x16_t& dp_c, f32x16_t& s_n,
                                           f32x16_t& dp_n, const bf16x8_t (&wp_p)[2], const bf16x8_t (&ws_p)[2],
                                           bf16x8_t (&wp_c)[2], bf16x8_t (&ws_c)[2], FusedOps& fo, const Dma& dma) {
  float nl[16];
  f32x16_t dinit, ninit;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const f32x4_t l4 = kUnit ? *(const lds_f32x4*)(nxt + 2 * kTileBytes + 4 * (32 * qbn + 8 * rr + 4 * g))
                             : *(const lds_f32x4*)(cur + 2 * kTileBytes + 4 * (32 * qb + 8 * rr + 4 * g));
    const f32x4_t d4 = *(const lds_f32x4*)(nxt + 2 * kTileBytes + 1024 + 4 * (32 * qbn + 8 * rr + 4 * g));
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      nl[4 * rr + qq] = l4[qq];
      ninit[4 * rr + qq] = l4[qq];
      dinit[4 * rr + qq] = d4[qq];
    }
  }
  s_n = kUnit ? ninit : f32x16_t{};
  dp_n = dinit;
  bf16x8_t op[32];
#pragma unroll
  for (int j = 0; j < kAhead; ++j)
    if (kPrev || (j & 1) == 0) op[j] = fused_operand(j, nxt, qbn, prv, qbp, a);
  __builtin_amdgcn_sched_barrier(0);
  float xa[16], p[16], x[16];
  uint32_t wpair[8], xpair[8];
#pragma unroll
  for (int k = 0; k < 34; ++k) {
    dma(k);
    if (k < 32) {
      const int kk = k + kAhead;
      if (kk < 32 && (kPrev || (kk & 1) == 0)) op[kk] = fused_operand(kk, nxt, qbn, prv, qbp, a);
      const int i = k >> 1;
      if ((k & 1) == 0) {
        if ((i & 1) == 0) s_n = mfma32(op[k], fo.kop[i >> 1], s_n);
        else dp_n = mfma32(op[k], fo.vop[i >> 1], dp_n);
      } else if (kPrev) {
        const int dblk = (i >> 1) & 3, jj = i >> 3;
        if ((i & 1) == 0) fo.dva[dblk] = mfma32(op[k], wp_p[jj], fo.dva[dblk]);
        else fo.dka[dblk] = mfma32(op[k], ws_p[jj], fo.dka[dblk]);
      }
    }
    if (!kUnit && k < 32 && (k & 1) == 0) xa[k >> 1] = fmaf(s_c[k >> 1], c, nl[k >> 1]);
    if (k < 32 && (k & 1) == 1) p[k >> 1] = __builtin_amdgcn_exp2f(kUnit ? s_c[k >> 1] : xa[k >> 1]);
    if (k >= 2 && k <= 32 && (k & 1) == 0) x[(k - 2) >> 1] = p[(k - 2) >> 1] * dp_c[(k - 2) >> 1];
    if (k >= 4 && k <= 32 && (k & 3) == 0) {
      const int m = (k - 4) >> 2;
      wpair[m] = pack_bf16x2(p[2 * m], p[2 * m + 1]);
    }
    if (k >= 5 && (k & 3) == 1) {
      const int m = (k - 5) >> 2;
      xpair[m] = pack_bf16x2(x[2 * m], x[2 * m + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    wp_c[h] = __builtin_bit_cast(bf16x8_t, u32x4_t{wpair[4 * h], wpair[4 * h + 1], wpair[4 * h + 2], wpair[4 * h + 3]});
    ws_c[h] = __builtin_bit_cast(bf16x8_t, u32x4_t{xpair[4 * h], xpair[4 * h + 1], xpair[4 * h + 2], xpair[4 * h + 3]});
  }
}

template <bool kUnit>
__global__ __launch_bounds__(64 * kFusedWaves, 1) void attention_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ stats, uint16_t* __restrict__ dk_out,
    uint16_t* __restrict__ dv_out, int L, int H, int Lp, float c, float scale, int n_full) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kFusedStages * kSlotBytes];
  int head, ktile;
  block_tile(blockIdx.x, H, n_full, head, ktile);
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tok_stride = (int64_t)H * kD;
  const int n_tiles = (L + kTile - 1) / kTile;
  const lds_char* lds = (const lds_char*)lds_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)lds_raw;
  const DmaOffsets<kFusedWaves> dmo = dma_offsets<kFusedWaves>(tok_stride, wave, lane);
  const uint16_t* qh = q + (int64_t)head * kD;
  const uint16_t* doh = dout + (int64_t)head * kD;
  const float* nlh = stats + (int64_t)head * Lp;
  const float* ndh = stats + ((int64_t)H + head) * Lp;
  // DMA piece j of tile t (clamped to the last tile: refetches keep the count
  // per step fixed): j = 0..3 Q, 4..7 dO, 8 a statistic -- -lse log2(e) from
  // even waves, -delta from odd ones (waves 2 and 3 repeat the identical
  // writes of waves 0 and 1, which keeps the step free of branches).
  const float* stat_src = (wave & 1) ? ndh : nlh;
  const uint32_t stat_off = 2 * kTileBytes + 1024 * (wave & 1);
  auto piece = [&](int t, int j) {
    const int tt = t < n_tiles ? t : n_tiles - 1;
    const uint32_t s = lds_base + (uint32_t)(t % kFusedStages) * kSlotBytes;
    if (j < 4) dma_row_piece<kFusedWaves>(qh, tok_stride, tt, L, dmo, s, wave, j);
    else if (j < 8) dma_row_piece<kFusedWaves>(doh, tok_stride, tt, L, dmo, s + kTileBytes, wave, j - 4);
    else dma_vec(stat_src, tt, Lp, s + stat_off, lane);
  };
  const auto slot = [&](int t) { return lds + (t % kFusedStages) * kSlotBytes; };
  static_assert(kFusedPieces == 8, "the step spreads eight row pieces over its slots");
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 9; ++j) piece(t, j);
  const int key = ktile * kFusedRows + wave * 32 + col;
  FusedOps fo;
  load_row_operands(k + (int64_t)head * kD, tok_stride, key, L, g, fo.kop);
  load_row_operands(v + (int64_t)head * kD, tok_stride, key, L, g, fo.vop);
  const Addr a = lds_addresses(lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) fo.dka[i] = fo.dva[i] = f32x16_t{};
  dma_wait();
  __syncthreads();

  // Block (0, 0)'s S and dP'.
  f32x16_t sa = f32x16_t{}, da, sb, db;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const f32x4_t d4 = *(const lds_f32x4*)(lds + 2 * kTileBytes + 1024 + 4 * (8 * rr + 4 * g));
    const f32x4_t l4 = *(const lds_f32x4*)(lds + 2 * kTileBytes + 4 * (8 * rr + 4 * g));
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      da[4 * rr + qq] = d4[qq];
      if (kUnit) sa[4 * rr + qq] = l4[qq];
    }
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    sa = mfma32(row_operand(lds, 0, ks, a), fo.kop[ks], sa);
    da = mfma32(row_operand(lds + kTileBytes, 0, ks, a), fo.vop[ks], da);
  }
  asm volatile("" : "+v"(sa), "+v"(da));
  // Block (t, 0) runs on set a (S, dP') and produces pa; block (t, 1) on set b, producing pb.
  bf16x8_t wpa[2], wsa[2], wpb[2], wsb[2];
  const auto no_dma = [](int) {};
  const auto wait_and_sync = [&]() {
    dma_wait_all_but<kFusedPieces + 1>();  // tile t + 1 landed; tile t + 2 may be in flight
    __syncthreads();
  };
  {
    const auto dma = [&](int kslot) {
      if ((kslot & 3) == 1 && kslot < 32) piece(2, kslot >> 2);
      if (kslot == 3) piece(2, 8);
    };
    fused_step<false, kUnit>(slot(0), 0, slot(0), 1, slot(0), 0, a, c, g, sa, da, sb, db, wpb, wsb, wpa, wsa, fo, dma);
    wait_and_sync();
  }
  // The last trip's second step, block (n_tiles, 0), finishes dV and dK of the
  // last block; its own scores come from a stale (loaded) slot and are never
  // used, like those of the next block in the first step of that trip.
  for (int t = 0; t < n_tiles; ++t) {
    fused_step<true, kUnit>(slot(t), 1, slot(t + 1), 0, slot(t), 0, a, c, g, sb, db, sa, da, wpa, wsa, wpb, wsb, fo,
                     no_dma);
    const auto dma = [&](int kslot) {
      if ((kslot & 3) == 1 && kslot < 32) piece(t + 3, kslot >> 2);
      if (kslot == 3) piece(t + 3, 8);
    };
    fused_step<true, kUnit>(slot(t + 1), 0, slot(t + 1), 1, slot(t), 1, a, c, g, sa, da, sb, db, wpb, wsb, wpa, wsa, fo,
                     dma);
    wait_and_sync();
  }
  dma_wait();
  if (key < L) {
    store_transposed(dk_out + (int64_t)key * tok_stride + (int64_t)head * kD, fo.dka, scale, g);
    store_transposed(dv_out + (int64_t)key * tok_stride + (int64_t)head * kD, fo.dva, 1.0f, g);
  }
}

}  // namespace

// An upper bound (for validation): every q-tile, plus up to 1024 run as two halves.
int64_t backward_grid_blocks(int64_t L, int32_t H) {
  const int64_t nfull = (L / kRows) * H;
  return ((L + kRows - 1) / kRows) * (int64_t)H + (nfull < 1024 ? nfull : 1024);
}
int64_t backward_workspace_bytes(int64_t L, int32_t H) { return 2 * (int64_t)H * ((L + kTile - 1) / kTile * kTile) * 4; }
int backward_block_threads() { return kThreads; }
// One past the last byte a row-tile DMA reads, from the tile's first byte (row
// kTile - 1, chunk 15); the offsets are 32-bit (see dma_offsets).
int64_t backward_tile_dma_end(int32_t H) { return (int64_t)(kTile - 1) * H * kD * 2 + kD * 2; }

// ---------------------------------------------------------------- scratch held by the library
// For callers that cannot allocate: the statistics buffer of the backward
// ([2][H][Lp] fp32) as a file-scope device array.  Every device that loads the
// library holds its own copy of kStaticScratchBytes until the process ends.  On
// the host, `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to a kernel.  All calls on a
// device share its copy; nothing in it needs clearing, since the dq kernel
// writes every statistic the dk/dv kernel then reads, in stream order.
constexpr int64_t kStaticScratchBytes = (int64_t)16 << 20;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int64_t backward_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t backward_static_scratch(int dev, float** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attention_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* out, const uint16_t* dout, const float* lse,
                                     uint16_t* dq, uint16_t* dk, uint16_t* dv, float* stats, int64_t L,
                                     int32_t H, float scale, hipStream_t stream) {
  const int n_half = forward_half_tiles(L, H);  // the same 256-row tiles, one workgroup per CU
  const dim3 grid((unsigned)(((L + kRows - 1) / kRows) * (int64_t)H + n_half)), block(kThreads);
  const int n_full = (int)(L / kRows);
  const int Lp = (int)((L + kTile - 1) / kTile * kTile);
  const float c = scale * kLog2e;
  if (c == 1.0f)
    hipLaunchKernelGGL(attention_bwd_dq_kernel<true>, grid, block, 0, stream, q, k, v, out, dout, lse, dq, stats,
                       (int)L, (int)H, Lp, c, scale, n_full, n_half);
  else
    hipLaunchKernelGGL(attention_bwd_dq_kernel<false>, grid, block, 0, stream, q, k, v, out, dout, lse, dq, stats,
                       (int)L, (int)H, Lp, c, scale, n_full, n_half);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid((unsigned)(((L + kFusedRows - 1) / kFusedRows) * (int64_t)H));
  if (c == 1.0f)
    hipLaunchKernelGGL(attention_bwd_dkdv_kernel<true>, fgrid, dim3(64 * kFusedWaves), 0, stream, q, k, v, dout,
                       stats, dk, dv, (int)L, (int)H, Lp, c, scale, (int)(L / kFusedRows));
  else
    hipLaunchKernelGGL(attention_bwd_dkdv_kernel<false>, fgrid, dim3(64 * kFusedWaves), 0, stream, q, k, v, dout,
                       stats, dk, dv, (int)L, (int)H, Lp, c, scale, (int)(L / kFusedRows));
  return hipGetLastError();
}

}  // namespace h3attn
