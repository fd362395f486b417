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
// head; each of its 4 waves owns 32 of them, and two workgroups share a CU (two
// waves per SIMD).  Keys stream through LDS in tiles of BN = 64.  Per tile a
// wave computes
//   S^T = K_tile * Q^T        (v_mfma_f32_32x32x16_bf16, 2 x 8)
//   softmax weights of S^T    (fp32; exp2 with scale*log2(e) folded into an FMA)
//   O^T += V_tile^T * P^T     (v_mfma_f32_32x32x16_bf16, 4 x 4)
// Computing the transposed score block makes each lane own one query column
// (lane % 32) and 16 keys of every 32-key block, so the fp32 accumulators of
// S^T convert in place to the bf16 B operand of the P*V product (no LDS round
// trip for P), and the row statistics need one cross-half exchange
// (v_permlane32_swap, no LDS).
//
// Software pipeline.  Iteration t issues
//   S(t+1) = K(t+1) Q^T        (matrix cores)
//   O += V(t-1)^T P(t-1)^T     (matrix cores)
//   P(t) = exp2(c S(t) - c m)  (VALU + transcendental unit)
// None of the three depends on another, so the 32 matrix instructions of an
// iteration are spread evenly through its ~100 vector instructions (the
// sched_group_barrier pattern below): a matrix instruction runs for 32 cycles,
// during which the same SIMD executes about three independent VALU
// instructions of this or of the other wave at no cost.
//
// LDS.  One 64 KiB array holds K and V tiles double-buffered: during iteration
// t the waves read K(t+1) and V(t-1) while DMA (buffer_load_dwordx4 ... lds,
// no VGPR staging) fills K(t+2) and V(t) into the other two buffers; one
// barrier per tile.  The buffers sit at fixed offsets, so the buffer choice
// folds into the ds_read immediate offset.  The DMA is issued by inline asm and
// awaited explicitly (vmcnt(0)) before each tile barrier: the compiler, which
// cannot prove that the in-flight writes miss the buffers being read, would
// otherwise wait for them before every LDS read.  Tiles are stored row-major
// (one 256-byte row per key, sixteen 16-byte chunks), chunk c of row r at
// physical chunk c ^ swz(r), swz(r) = 4*(r & 3) + ((r >> 2) & 3).  The LDS has
// 64 four-byte banks and serves 16 lanes of a 16-byte read, or 32 lanes of an
// 8-byte read, per cycle; swz takes 16 distinct values over any 16 consecutive
// rows (the K operand read) and distinct top bits over 4 consecutive rows (the
// transposed V read, ds_read_b64_tr_b16: 32 lanes = 4 keys x 4 chunks), so
// both are conflict-free (checked with the SQ_LDS_BANK_CONFLICT counter).
//
// Exponent offset.  The weights of a tile are computed against the offset m
// the row already has, with no per-tile maximum.  Each lane adds up the bf16
// weights it produced (v_dot2_f32_bf16 against (1, 1): exactly the values that
// enter the P*V product, so O / l does not depend on m).  If some lane's sum
// exceeds 2^8 (so some weight may exceed 2^8, or overflowed), the wave takes a
// rare path: m moves to the row maximum of the tile, the already accumulated O
// and l are scaled by 2^(c (m_old - m_new)), and the tile's weights are
// recomputed.  m starts at -FLT_MAX, so the first tile always takes that path.
// Every weight that reaches the matrix cores is therefore at most 2^8.
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "h3attn_internal.h"

namespace h3attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;

constexpr int kD = 128;
constexpr int kBM = 128;                  // query rows per workgroup
constexpr int kBN = 64;                   // keys per tile
constexpr int kThreads = 256;
constexpr int kTileBytes = kBN * kD * 2;  // 16 KiB per K or V tile
constexpr int kK0 = 0, kK1 = kTileBytes, kV0 = 2 * kTileBytes, kV1 = 3 * kTileBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSumBound = 256.0f;        // a lane's tile sum of P above this moves the offset

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;  // v_cvt_pk_bf16_f32: round to nearest even
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Reduce over the lane pair (l, l ^ 32): with both operands = x, the swap
// returns x of the lower half and x of the upper half in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Byte offset of (row, channel) in a swizzled tile; channel % 4 == 0.
__device__ __forceinline__ int tile_offset(int row, int ch) {
  return row * (kD * 2) + ((((ch >> 3) ^ swz(row))) << 4) + ((ch & 7) << 1);
}

// ---------------------------------------------------------------- tile DMA
// One 64-key tile of a [L][H][128] tensor goes into a swizzled LDS tile as 16
// pieces of 1 KiB; wave w writes pieces w, w+4, w+8, w+12.  A piece is 64
// lanes x 16 bytes in lane order at M0; lane `lane` fetches the global chunk
// that belongs at its slot, at a fixed byte offset from the tile base.  The
// load goes through a buffer resource whose size ends at the document's last
// row: rows past it read as zeros (their scores are masked to -inf and their
// V rows then contribute nothing), and no address outside the tensor is used.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;  // raw buffer, 32-bit data format

struct DmaOffsets {
  uint32_t off[4];
};

__device__ __forceinline__ DmaOffsets dma_offsets(int64_t tok_stride, int wave, int lane) {
  DmaOffsets d;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int slot = (it * 4 + wave) * 64 + lane;  // 16-byte slot in the tile
    const int r = slot >> 4;
    const int c = (slot & 15) ^ swz(r);
    d.off[it] = (uint32_t)(((int64_t)r * tok_stride + 8 * c) * 2);
  }
  return d;
}

// tile_base: first byte of the tile's row 0 (this head); valid_bytes: bytes
// from there to the end of the document's last row of this head.
__device__ __forceinline__ void tile_dma(const char* tile_base, int64_t valid_bytes, const DmaOffsets& d,
                                         uint32_t lds_tile, int wave) {
  const uint64_t b = (uint64_t)(uintptr_t)tile_base;
  const uint32_t n = valid_bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)valid_bytes;
  const i32x4_t rsrc = {(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
                        (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)),
                        (int)__builtin_amdgcn_readfirstlane(n), kBufferDword3};
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_tile + (it * 4 + wave) * 1024);
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(d.off[it]), "s"(m0), "s"(rsrc)
                 : "memory");
  }
}

// All of this wave's tile DMA has landed in LDS.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Keeps the compiler from flattening a rarely taken branch into straight-line
// selects executed on every tile.
__device__ __forceinline__ void cold_path() { asm volatile("" ::: "memory"); }


// ---------------------------------------------------------------- per-wave state
struct State {
  bf16x8_t q[8];   // Q^T operand: q[ks] = Q[row][16 ks + 8 g .. +7]
  f32x16_t o[4];   // O^T accumulators, d-blocks of 32
  float m;         // exponent offset (raw score units)
  float l;         // this lane-half's partial sum of P
};

// LDS read addresses.  With the swizzle above, the k-step of a K read and the
// d-block of a V read enter the byte offset through bits that no other term
// touches, so each read address is a per-lane base XOR a constant (plus an
// immediate for the 32-key block, the 16-key step and the buffer):
//   K (row 32 kb + col, channels 16 ks + 8 g .. +7):
//     kb * 8192 + (kaddr ^ 32 ks),  kaddr = 256 col + (16 g ^ 16 swz(col))
//   V (row 16 j + 8 h + key_a, channels 32 dblk + ch .. +3):
//     4096 j + (vaddr[h] ^ 64 dblk),
//     vaddr[h] = 256 (8 h + key_a) + 8 ((ch >> 2) & 1) + (16 (ch >> 3) ^ 16 swz(8 h + key_a))
// The bases are refreshed opaquely each iteration so the compiler derives the
// addresses with one XOR each instead of keeping 28 of them live.
struct Addr {
  uint32_t k, v0, v1;
};

// One MFMA of S^T = K_tile Q^T: 32-key block kb, k-step ks.
template <int kBuf>
__device__ __forceinline__ void qk_step(f32x16_t& s, int kb, int ks, const State& st, const lds_char* lds,
                                        const Addr& a) {
  const bf16x8_t op = *(const lds_bf16x8*)(lds + kBuf + kb * 8192 + (a.k ^ (32u * ks)));
  s = mfma32(op, st.q[ks], s);
}

// One MFMA of O^T += V_tile^T P^T: d-block dblk, 16-key step j.  The A operand
// comes from two transposed reads: lane l (group G = l >> 4, index i = l & 15)
// addresses key 16 j + 4 (G >> 1) + (i >> 2) (+8 for the second read) at
// channel 32 dblk + 16 (G & 1) + 4 (i & 3), and receives keys {16 j + 4 g + e}
// and {16 j + 8 + 4 g + e} of channel 32 dblk + (l % 32) -- the key order of
// the P^T accumulator slots.
template <int kBuf>
__device__ __forceinline__ void pv_step(State& st, int dblk, int j, const bf16x8_t (&p)[4], const lds_char* lds,
                                        const Addr& a) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + kBuf + 4096 * j + (a.v0 ^ (64u * dblk))));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + kBuf + 4096 * j + (a.v1 ^ (64u * dblk))));
  const i16x8_t a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  st.o[dblk] = mfma32(__builtin_bit_cast(bf16x8_t, a16), p[j], st.o[dblk]);
}

template <int kBuf>
__device__ __forceinline__ void pv(State& st, const bf16x8_t (&p)[4], const lds_char* lds, const Addr& a) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) pv_step<kBuf>(st, dblk, j, p, lds, a);
}

// Weights of score pair i (i = 0..15: block kb = i / 8, slots 2 (i % 8), +1)
// against offset mc = c m: P = 2^(c s - mc), rounded to bf16 for the P*V
// product; the lane sum adds the same rounded values (v_dot2_f32_bf16 against
// (1, 1)) into one of four partial sums.
__device__ __forceinline__ void weight_pair(const f32x16_t (&s)[2], int i, float c, float mc, bf16x8_t (&p)[4],
                                            float (&ps)[4]) {
  const int kb = i >> 3, e = 2 * (i & 7);
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x2_t pr;
  pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][e], c, -mc));
  pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][e + 1], c, -mc));
  ps[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps[i & 3], false);
  p[2 * kb + (e >> 3)][e & 7] = pr[0];
  p[2 * kb + (e >> 3)][(e & 7) + 1] = pr[1];
}

// Rare path: move the offset to the row maximum of this tile (or keep it if
// larger), scale O and l to the new offset and recompute the tile's weights.
// Runs after this iteration's P*V product, which used the old offset.
__device__ __forceinline__ float rebase(const f32x16_t (&s_in)[2], State& st, float c, bf16x8_t (&p)[4]) {
  // An opaque copy: keeps the compiler from hoisting this path's arithmetic
  // into the common path in front of the branch.
  f32x16_t s[2] = {s_in[0], s_in[1]};
  asm volatile("" : "+v"(s[0]), "+v"(s[1]));
  float m0 = fmaxf(s[0][0], s[0][1]);
  float m1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int e = 2; e < 16; e += 2) {
    m0 = fmaxf(fmaxf(m0, s[0][e]), s[0][e + 1]);
    m1 = fmaxf(fmaxf(m1, s[1][e]), s[1][e + 1]);
  }
  // Both lane-halves of a query see the same maximum and so the same offset.
  const float m_new = fmaxf(st.m, pair_max(fmaxf(m0, m1)));
  const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * c);  // 0 on the first tile
  st.m = m_new;
  st.l *= alpha;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.o[i] *= alpha;
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
  const float mc = m_new * c;
#pragma unroll
  for (int i = 0; i < 16; ++i) weight_pair(s, i, c, mc, p, ps);
  return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

// Scores of keys at or past L (only in the last, partial tile) become -inf.
__device__ __forceinline__ void mask_tail(f32x16_t (&s)[2], int kbase, int L, int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        if (kbase + 32 * kb + 8 * r + 4 * g + qq >= L) s[kb][4 * r + qq] = -INFINITY;
}

// ---------------------------------------------------------------- kernel
struct Ctx {
  const lds_char* lds;
  uint32_t lds_base;
  const char* kbase;
  const char* vbase;
  int64_t tile_stride_bytes;  // 64 rows
  int64_t row_bytes;          // one token row of all heads
  DmaOffsets dma;
  int n_full, n_tiles, L, wave, g;
  float c;
};

__device__ __forceinline__ void dma(const Ctx& x, const char* base, int t, int buf) {
  const int64_t valid = (int64_t)(x.L - 1 - t * kBN) * x.row_bytes + kD * 2;
  tile_dma(base + t * x.tile_stride_bytes, valid, x.dma, x.lds_base + buf, x.wave);
}

// The 32 matrix instructions of an iteration, in issue order ("slots"): even
// slot k is score MFMA k/2 (block kb = (k/2) & 1, k-step ks = k/4), odd slot k
// is P*V MFMA (k-1)/2 (16-key step j = k/8, d-block (k/2) & 3).  Chains of
// dependent MFMAs are 4 (scores) or 8 (P*V) slots apart.
template <int kKNext, int kVPrev>
__device__ __forceinline__ bf16x8_t slot_operand(int k, const lds_char* lds, const Addr& a) {
  const int i = k >> 1;
  if ((k & 1) == 0) return *(const lds_bf16x8*)(lds + kKNext + (i & 1) * 8192 + (a.k ^ (32u * (i >> 1))));
  const int j = i >> 2, dblk = i & 3;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + kVPrev + 4096 * j + (a.v0 ^ (64u * dblk))));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + kVPrev + 4096 * j + (a.v1 ^ (64u * dblk))));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Iteration t: S(t+1) from K(t+1) in buffer kKNext into s_next; O += V(t-1)
// P(t-1) from buffer kVPrev (skipped for t = 0); P(t) from s_cur into p_cur.
// DMA fills K(t+2) into kKFill (when it exists) and V(t) into kVFill.  In the
// last iteration there is no K(t+1): S(t+1) is computed from the stale buffer
// and never used.
//
// With the P*V product (t > 0) the instruction order is fixed by hand, slot by
// slot, with scheduling barriers in between: the operand reads of slot k + 2,
// the MFMA of slot k, then a share of the weights -- the two FMAs of score
// pair k/2 on even slots (plus the bf16 pack and row-sum of pair k/2 - 1), the
// two exponentials of pair k/2 on odd slots.  Each slot then holds about one
// MFMA's worth (32 cycles) of vector work, and every dependency is at least one
// MFMA apart.
template <int kKNext, int kVPrev, int kKFill, int kVFill, bool kPV>
__device__ __forceinline__ void iteration(const Ctx& x, State& st, Addr& a, const f32x16_t (&s_cur)[2],
                                          f32x16_t (&s_next)[2], const bf16x8_t (&p_prev)[4],
                                          bf16x8_t (&p_cur)[4], int t) {
  asm volatile("" : "+v"(a.k), "+v"(a.v0), "+v"(a.v1));
  if (t + 2 < x.n_tiles) dma(x, x.kbase, t + 2, kKFill);
  dma(x, x.vbase, t, kVFill);

  const float c = x.c, mc = st.m * c;
  float ps[4] = {0.f, 0.f, 0.f, 0.f};
  s_next[0] = f32x16_t{};
  s_next[1] = f32x16_t{};
  if (kPV) {
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float xa[16], xb[16];
    bf16x8_t op[32];
    op[0] = slot_operand<kKNext, kVPrev>(0, x.lds, a);
    op[1] = slot_operand<kKNext, kVPrev>(1, x.lds, a);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k + 2 < 32) op[k + 2] = slot_operand<kKNext, kVPrev>(k + 2, x.lds, a);
      const int i = k >> 1;
      if ((k & 1) == 0) {
        s_next[i & 1] = mfma32(op[k], st.q[i >> 1], s_next[i & 1]);
      } else {
        st.o[i & 3] = mfma32(op[k], p_prev[i >> 2], st.o[i & 3]);
      }
      const int kb = i >> 3, e = 2 * (i & 7);  // score pair i = k/2
      if ((k & 1) == 0) {
        xa[i] = fmaf(s_cur[kb][e], c, -mc);
        xb[i] = fmaf(s_cur[kb][e + 1], c, -mc);
        if (i > 0) {
          const int kb1 = (i - 1) >> 3, e1 = 2 * ((i - 1) & 7);
          bf16x2_t pr;
          pr[0] = (__bf16)xa[i - 1];
          pr[1] = (__bf16)xb[i - 1];
          ps[(i - 1) & 3] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps[(i - 1) & 3], false);
          p_cur[2 * kb1 + (e1 >> 3)][e1 & 7] = pr[0];
          p_cur[2 * kb1 + (e1 >> 3)][(e1 & 7) + 1] = pr[1];
        }
      } else {
        xa[i] = __builtin_amdgcn_exp2f(xa[i]);
        xb[i] = __builtin_amdgcn_exp2f(xb[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x2_t pr;
    pr[0] = (__bf16)xa[15];
    pr[1] = (__bf16)xb[15];
    ps[3] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps[3], false);
    p_cur[3][6] = pr[0];
    p_cur[3][7] = pr[1];
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s_next[kb] = mfma32(slot_operand<kKNext, kVPrev>(4 * ks + 2 * kb, x.lds, a), st.q[ks], s_next[kb]);
#pragma unroll
    for (int i = 0; i < 16; ++i) weight_pair(s_cur, i, c, mc, p_cur, ps);
  }
  float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  if (__builtin_amdgcn_ballot_w64(!(psum <= kSumBound)) != 0) {
    cold_path();
    psum = rebase(s_cur, st, c, p_cur);
  }
  st.l += psum;
  if (t + 1 >= x.n_full) {
    cold_path();
    mask_tail(s_next, (t + 1) * kBN, x.L, x.g);
  }
  dma_wait();
  __syncthreads();  // K(t+2), V(t) landed; every wave is done with K(t+1), V(t-1)
}

__global__ __launch_bounds__(kThreads, 2) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, int L, int H, float scale_log2e, int n_qtiles) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[4 * kTileBytes];

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
  Ctx x;
  x.lds = (const lds_char*)lds_raw;
  x.lds_base = (uint32_t)(uintptr_t)(lds_char*)lds_raw;
  x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  x.g = lane >> 5;
  x.L = L;
  x.c = scale_log2e;
  const int64_t tok_stride = (int64_t)H * kD;      // elements between consecutive tokens
  x.row_bytes = tok_stride * 2;
  x.n_full = L / kBN;                              // tiles with 64 real keys
  x.n_tiles = (L + kBN - 1) / kBN;                 // plus one partial tile if L % 64 != 0
  x.tile_stride_bytes = (int64_t)kBN * x.row_bytes;
  x.kbase = reinterpret_cast<const char*>(k + (int64_t)head * kD);
  x.vbase = reinterpret_cast<const char*>(v + (int64_t)head * kD);
  x.dma = dma_offsets(tok_stride, x.wave, lane);

  Addr a;
  a.k = 256u * col + ((16u * x.g) ^ (16u * swz(col)));
  {
    const int key_a = 4 * (lane >> 5) + ((lane & 15) >> 2);  // transposed-read key of this lane
    const int ch = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // transposed-read channel
    a.v0 = 256u * key_a + 8u * ((ch >> 2) & 1) + ((16u * (ch >> 3)) ^ (16u * swz(key_a)));
    a.v1 = 256u * (8 + key_a) + 8u * ((ch >> 2) & 1) + ((16u * (ch >> 3)) ^ (16u * swz(8 + key_a)));
  }

  dma(x, x.kbase, 0, kK0);
  if (x.n_tiles > 1) dma(x, x.kbase, 1, kK1);

  // Q^T operand: lane holds Q[row][16ks + 8g .. +7] for its query row.
  State st;
  const int qrow = qtile * kBM + x.wave * 32 + col;
  if (qrow < L) {
    const uint16_t* p = q + (int64_t)qrow * tok_stride + (int64_t)head * kD + 8 * x.g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st.q[ks] = *reinterpret_cast<const bf16x8_t*>(p + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st.q[ks] = bf16x8_t{};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) st.o[i] = f32x16_t{};
  st.m = -FLT_MAX;
  st.l = 0.f;
  dma_wait();
  __syncthreads();  // K(0), K(1) are in LDS

  f32x16_t s0[2], s1[2];
  bf16x8_t p0[4], p1[4];
  s0[0] = f32x16_t{};
  s0[1] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qk_step<kK0>(s0[0], 0, ks, st, x.lds, a);
    qk_step<kK0>(s0[1], 1, ks, st, x.lds, a);
  }
  if (x.n_full == 0) mask_tail(s0, 0, L, x.g);
  // The first iteration refills buffer K0 with K(2): every wave must be done
  // reading K(0) first.  (Later refills are ordered by the previous
  // iteration's barrier.)
  __syncthreads();

  // Iteration t reads K(t+1) from buffer (t+1)%2 and V(t-1) from buffer
  // (t-1)%2; S(t) and P(t) live in s/p[t%2].  Odd/even pairs keep the buffer
  // choice static.
  iteration<kK1, kV1, kK0, kV0, false>(x, st, a, s0, s1, p1, p0, 0);
  int t = 1;
  for (; t + 1 < x.n_tiles; t += 2) {
    iteration<kK0, kV0, kK1, kV1, true>(x, st, a, s1, s0, p0, p1, t);
    iteration<kK1, kV1, kK0, kV0, true>(x, st, a, s0, s1, p1, p0, t + 1);
  }
  if (t < x.n_tiles) {
    iteration<kK0, kV0, kK1, kV1, true>(x, st, a, s1, s0, p0, p1, t);
    pv<kV1>(st, p1, x.lds, a);  // P(t) V(t), t odd
  } else {
    pv<kV0>(st, p0, x.lds, a);  // P(t-1) V(t-1), t-1 even
  }

  // Epilogue: full row sum = both lane-halves; O / l -> bf16.
  const float inv_l = 1.0f / pair_sum(st.l);
  if (qrow < L) {
    uint16_t* po = out + (int64_t)qrow * tok_stride + (int64_t)head * kD;
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * dblk + 8 * r + 4 * x.g;
        *reinterpret_cast<uint2*>(po + d) =
            make_uint2(pack_bf16x2(st.o[dblk][4 * r] * inv_l, st.o[dblk][4 * r + 1] * inv_l),
                       pack_bf16x2(st.o[dblk][4 * r + 2] * inv_l, st.o[dblk][4 * r + 3] * inv_l));
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
