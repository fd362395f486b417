// Full bidirectional (non-causal, unmasked) flash attention forward for gfx950.
//
// Operation ("MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 2 "Attention:
// full bidirectional self-attention"; section 4 "Full attention is non-causal
// and unmasked over one packed document"; section 5 item h3_full_attention):
//   out[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k[j,h,:]>) v[j,h,:]
//
// One kernel template, four instantiations.  The plain one computes exactly
// that, with the scale applied in fp32 to each score.  The log2 one expects q to carry
// scale * log2(e) already (the Q/K prologue applies it in fp32 before q's
// single rounding to bf16, so q is rounded once either way) and computes
//   out[i,h,:] = sum_j 2^<q[i,h,:], k[j,h,:]> v[j,h,:] / sum_j 2^<q[i,h,:], k[j,h,:]>
// which is the same softmax: its scores come out of the matrix cores in the
// exponent's units, and the offset is subtracted there too (the score MFMA
// chain starts from -m instead of 0), so no vector instruction stands between
// a score and its exponential.  Two more forms build on the log2 one: the Q
// prologue form takes the raw q and applies Q's RMSNorm and MM-RoPE (with
// gamma_q, the rotation table K's prologue wrote and the factor scale log2(e))
// at its Q load, with the standalone prologue's fp32 operations and rounding;
// the quantized-score form, on top of that, computes the scores from e4m3
// operands (4 q' in registers, K' / 4 as bytes from its own K prologue) on the
// FP8 matrix instruction, a cast its entry point declares.
//
// Numerical contract (same RFC, section 4): fp32 accumulation on the matrix
// cores, one fixed key order (tile 0, 1, 2, ...), no split over keys, no
// atomics; every output row is produced by exactly one wave, so the result
// does not depend on the grid or on the number of CUs.
//
// Work decomposition.  A 512-thread workgroup owns BM = 256 query rows of one
// head; each of its 8 waves owns 32 of them (two waves per SIMD, one workgroup
// per CU).  Keys stream through LDS in tiles of BN = 64, shared by all 8
// waves.  Per tile a wave computes
//   S^T = K_tile * Q^T        (v_mfma_f32_32x32x16_bf16, 2 x 8)
//   softmax weights of S^T    (fp32; exp2 with scale*log2(e) folded into an FMA)
//   O^T += V_tile^T * P^T     (v_mfma_f32_32x32x16_bf16, 4 x 4)
// Computing the transposed score block makes each lane own one query column
// (lane % 32) and 16 keys of every 32-key block, so the fp32 accumulators of
// S^T convert in place to the bf16 B operand of the P*V product (no LDS round
// trip for P), and the row statistics need one cross-half exchange
// (v_permlane32_swap, no LDS).
//
// Key order.  The B operand of a 32x32x16 MFMA takes k-slots 8g .. 8g+7 from
// lane half g; the P^T operand built from S^T accumulator rows holds, in those
// slots, keys 16j + {4g .. 4g+3, 8+4g .. 11+4g}.  The plain variant gathers the
// V^T operand from the row-major V tile in that same key order by two
// transposing LDS reads (ds_read_b64_tr_b16).  The log2 variant reads V
// transposed ([H][128][Lp] in memory, so a tile is 128 channel rows of 64 keys)
// with one 16-byte read of 8 consecutive keys, and permutes the rows of its K
// tile instead (bits 2 and 3 of the row index swapped), which makes the P^T
// slots of a lane half hold consecutive keys.  No data is reordered anywhere.
//
// Software pipeline.  Iteration t issues
//   S(t+1) = K(t+1) Q^T        (matrix cores)
//   O += V(t-1)^T P(t-1)^T     (matrix cores)
//   P(t) = exp2(c S(t) - c m)  (VALU + transcendental unit)
// None of the three depends on another, so the 32 matrix instructions of an
// iteration are spread evenly through its ~100 vector instructions: a matrix
// instruction runs for 32 cycles, during which the same SIMD executes about
// three independent VALU instructions of this or of the other wave at no cost.
//
// LDS.  Two rings of four 16 KiB tiles, K and V (128 KiB): during iteration t
// the waves read K(t+1) and V(t-1) while DMA (buffer_load_dwordx4 ... lds, no
// VGPR staging) fills K(t+4) and V(t+2), each into the slot its ring freed in
// iteration t-1; one barrier per tile, and a DMA has about two iterations to
// land.  The tile descriptors advance by one tile per iteration.  The DMA is
// issued by inline asm and awaited explicitly (vmcnt) before
// each tile barrier: the compiler, which cannot prove that the in-flight writes
// miss the buffers being read, would otherwise wait for them before every LDS
// read.  Row-major tiles (one 256-byte row per key, sixteen 16-byte chunks)
// put chunk c of row r at physical chunk c ^ swz(r),
// swz(r) = 4 (r & 3) + ((r >> 2) & 3); V^T tiles (128-byte rows) put chunk c
// of row d at c ^ ((d >> 1) & 7).  The LDS has 64 four-byte banks and serves
// 16 lanes of a 16-byte read, or 32 lanes of an 8-byte read, per cycle; both
// swizzles spread each read over all banks, so every operand read is
// conflict-free (checked with the SQ_LDS_BANK_CONFLICT counter).
//
// Exponent offset.  The weights of a tile are computed against the offset m
// the row already has, with no per-tile maximum.  Each lane adds up the bf16
// weights it produced (exactly the values that enter the P*V product, so O / l
// does not depend on m; a sum of the fp32 weights before rounding would not
// cancel their rounding when a few keys dominate a row).  If some lane's sum
// exceeds 2^8 (so some weight may exceed 2^8, or overflowed), the wave takes a
// rare path: m moves to the row maximum of the tile, the already accumulated O
// and l are scaled by 2^(m_old - m_new) in exponent units, and the tile's
// weights are recomputed.  Every weight that reaches the matrix cores is
// therefore at most 2^8.  The plain variant starts m at -FLT_MAX, so its first
// tile always takes that path; the log2 variant starts m at the first tile's
// row maximum.
//
// Grid order.  Each head's partial last q-tile (L not a multiple of 256) is
// dispatched last, and its waves that own no query row only carry their share
// of the DMA, so those shorter workgroups fill the grid's final round.
#include <hip/hip_runtime.h>

#include <atomic>
#include <float.h>
#include <stdint.h>

#include "gfx950_tile.h"
#include "h3attn_internal.h"

namespace h3attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;                 // waves per workgroup, 32 query rows each
constexpr int kBM = 32 * kWaves;          // query rows per workgroup
constexpr int kBN = 64;                   // keys per tile
constexpr int kThreads = 64 * kWaves;
constexpr int kDmaPerWave = 16 / kWaves;  // 1 KiB DMA pieces per wave per tile
static_assert(kDmaPerWave == 2, "the slot loop issues two K and two V pieces per wave");
constexpr int kTileBytes = kBN * kD * 2;  // 16 KiB per K or V tile
constexpr int kStages = 4;                // tiles per ring (resident or in flight)
constexpr int kVRing = kStages * kTileBytes;  // the V ring follows the K ring
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSumBound = 256.0f;        // a lane's tile sum of P above this moves the offset

__device__ __forceinline__ int vswz(int row) { return (row >> 1) & 7; }
// Key held by row r of a K tile (and by S^T accumulator row r) when V comes
// transposed: bits 2 and 3 of r swapped.
__device__ __forceinline__ int perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ---------------------------------------------------------------- tile DMA
// A 64-key tile of a [L][H][128] tensor goes into LDS as 16 pieces of 1 KiB;
// wave w writes pieces w and w+8.  A piece is 64 lanes x 16 bytes in lane order
// at M0; each lane fetches the global chunk that belongs at its slot, at a fixed
// byte offset from the tile base.  Loads go through a buffer resource whose size
// ends at the document's last row: rows past it read as zeros (their scores are
// masked to -inf and their V rows then contribute nothing), and no address
// outside the tensor is used.
struct DmaOffsets {
  uint32_t off[kDmaPerWave];
};

// Row-major tile: slot (row r, physical chunk p) <- token r (token perm(r)
// with kPerm) of the tile, channels 8 (p ^ swz(r)) .. +7.
template <bool kPerm>
__device__ __forceinline__ DmaOffsets dma_offsets(int64_t tok_stride, int wave, int lane) {
  DmaOffsets d;
#pragma unroll
  for (int it = 0; it < kDmaPerWave; ++it) {
    const int slot = (it * kWaves + wave) * 64 + lane;  // 16-byte slot in the tile
    const int r = slot >> 4;
    const int c = (slot & 15) ^ swz(r);
    d.off[it] = (uint32_t)(((int64_t)(kPerm ? perm(r) : r) * tok_stride + 8 * c) * 2);
  }
  return d;
}

// V^T tile (128 channel rows of 64 keys, 128 bytes): slot (row d, physical
// chunk p) <- channel d, keys 8 (p ^ vswz(d)) .. +7.
__device__ __forceinline__ DmaOffsets vt_dma_offsets(int64_t vt_row_bytes, int wave, int lane) {
  DmaOffsets d;
#pragma unroll
  for (int it = 0; it < kDmaPerWave; ++it) {
    const int slot = (it * kWaves + wave) * 64 + lane;
    const int r = slot >> 3;
    const int c = (slot & 7) ^ vswz(r);
    d.off[it] = (uint32_t)(r * vt_row_bytes + 16 * c);
  }
  return d;
}

// K8 tile (the FP8 variant: 64 key rows of 128 bytes, the log2 variant's row
// permutation): one 1 KiB piece per wave; slot (row r, physical chunk p) <- key
// perm(r), bytes 16 (p ^ vswz(r)) .. +15.
__device__ __forceinline__ DmaOffsets k8_dma_offsets(int64_t row_bytes, int wave, int lane) {
  DmaOffsets d;
  const int slot = wave * 64 + lane;
  const int r = slot >> 3;
  const int c = (slot & 7) ^ vswz(r);
  d.off[0] = d.off[1] = (uint32_t)(perm(r) * row_bytes + 16 * c);
  return d;
}

// A tile's DMA: the buffer resource (tile_base: first byte of the tile;
// valid_bytes: bytes from there to the end of the valid data) and this wave's
// LDS destination (the tile's LDS offset plus its first piece).
struct TileDma {
  i32x4_t rsrc;
  uint32_t lds;
};

__device__ __forceinline__ TileDma tile_dma(const char* tile_base, int64_t valid_bytes, uint32_t lds_tile,
                                            int wave) {
  const uint64_t b = (uint64_t)(uintptr_t)tile_base;
  // valid_bytes > 0 here; past 2^32 - 1 the record count saturates (a 32-bit
  // test of the high word: there is no 64-bit scalar less-than).
  const uint32_t n = (uint32_t)((uint64_t)valid_bytes >> 32) != 0u ? 0xffffffffu : (uint32_t)valid_bytes;
  TileDma t;
  t.rsrc = i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
                   (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)),
                   (int)__builtin_amdgcn_readfirstlane(n), kBufferDword3};
  t.lds = __builtin_amdgcn_readfirstlane(lds_tile + wave * 1024);
  return t;
}

// Issue this wave's DMA piece it (0 .. kDmaPerWave-1) of a tile.
__device__ __forceinline__ void dma_piece(const TileDma& t, const DmaOffsets& d, int it) {
  lds_dma_dwordx4(t.rsrc, d.off[it], t.lds + it * kWaves * 1024);
}

__device__ __forceinline__ void dma_all(const TileDma& t, const DmaOffsets& d) {
#pragma unroll
  for (int it = 0; it < kDmaPerWave; ++it) dma_piece(t, d, it);
}

// Keeps the compiler from flattening a rarely taken branch into straight-line
// selects executed on every tile.
__device__ __forceinline__ void cold_path() { asm volatile("" ::: "memory"); }

// ---------------------------------------------------------------- per-wave state
struct State {
  bf16x8_t q[8];   // Q^T operand: q[ks] = Q[row][16 ks + 8 g .. +7]
  i32x8_t q8[2];   // FP8 variant: the same 64 values, times 4, as e4m3 (k-steps of 64)
  f32x16_t o[4];   // O^T accumulators, d-blocks of 32
  f32x16_t minit;  // log2 variant: -m in every slot, the score chain's start
  float m;         // exponent offset (raw score units; log2 variant: log2 units)
  float l;         // this lane-half's partial sum of P
  // The K tile this iteration's DMA fetches (tile t + kStages, clamped to the
  // last): its first byte and the valid bytes from there, advanced by one tile
  // per iteration instead of recomputed from t (a 64-bit product per tile).
  const char* kt_base;
  int64_t kt_valid;
  const char* vt_base;  // the same for the V (or V^T) tile, tile t + kStages - 2
  int64_t vt_valid;
};

// LDS read addresses.  With the swizzle above, the k-step of a K read and the
// d-block of a V read enter the byte offset through bits that no other term
// touches, so each read address is a per-lane base XOR a constant, plus an
// immediate for the 32-key block or the 16-key step:
//   K (row 32 kb + col, channels 16 ks + 8 g .. +7):
//     kb * 8192 + (kaddr ^ 32 ks),  kaddr = buf + 256 col + (16 g ^ 16 swz(col))
//   V (row 16 j + 8 h + key_a, channels 32 dblk + ch .. +3):
//     4096 j + (vaddr[h] ^ 64 dblk),
//     vaddr[h] = buf + 256 (8 h + key_a) + 8 ((ch >> 2) & 1) + (16 (ch >> 3) ^ 16 swz(8 h + key_a))
// The buffer offset buf is a multiple of 16 KiB and does not meet the XOR.
struct Addr {
  uint32_t k, v0, v1;
};

__device__ __forceinline__ Addr at_buffers(const Addr& a, uint32_t kbuf, uint32_t vbuf) {
  return Addr{a.k + kbuf, a.v0 + vbuf, a.v1 + vbuf};
}

// Operand of the score MFMA for 32-key block kb, k-step ks.
__device__ __forceinline__ bf16x8_t k_operand(int kb, int ks, const lds_char* lds, const Addr& b) {
  return *(const lds_bf16x8*)(lds + kb * 8192 + (b.k ^ (32u * ks)));
}

// FP8 variant: operand of the score MFMA (k = 64) for 32-key block kb, k-step
// ks: bytes 64 g + 32 ks .. +31 of key row 32 kb + col of the K8 tile (128-byte
// rows, chunk c of row r at c ^ vswz(r), as a V^T tile), in two 16-byte reads;
// the per-lane base is kaddr = buf + 128 col + 16 (4 g ^ vswz(col)).
__device__ __forceinline__ i32x8_t k8_operand(int kb, int ks, const lds_char* lds, const Addr& b) {
  const i32x4_t lo = __builtin_bit_cast(i32x4_t, *(const lds_bf16x8*)(lds + kb * 4096 + (b.k ^ (32u * ks))));
  const i32x4_t hi = __builtin_bit_cast(i32x4_t, *(const lds_bf16x8*)(lds + kb * 4096 + (b.k ^ (32u * ks + 16u))));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand of the P*V MFMA for d-block dblk, 16-key step j: two transposing
// reads.  Lane l (group G = l >> 4, index i = l & 15) addresses key
// 16 j + 4 (G >> 1) + (i >> 2) (+8 for the second read) at channel
// 32 dblk + 16 (G & 1) + 4 (i & 3), and receives keys {16 j + 4 g + e} and
// {16 j + 8 + 4 g + e} of channel 32 dblk + (l % 32) -- the key order of the
// P^T accumulator slots.
template <bool kVT>
__device__ __forceinline__ bf16x8_t v_operand(int dblk, int j, const lds_char* lds, const Addr& b) {
  // From a V^T tile: one 16-byte read at row 32 dblk + col, keys 16 j + 8 g .. +7.
  if (kVT) return *(const lds_bf16x8*)(lds + dblk * 4096 + (b.v0 ^ (32u * j)));
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + 4096 * j + (b.v0 ^ (64u * dblk))));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + 4096 * j + (b.v1 ^ (64u * dblk))));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// O^T += V_tile^T P^T.
template <bool kVT>
__device__ __forceinline__ void pv(State& st, const bf16x8_t (&p)[4], const lds_char* lds, const Addr& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) st.o[dblk] = mfma32(v_operand<kVT>(dblk, j, lds, b), p[j], st.o[dblk]);
}

// Weights.  Score n (0..31) of a lane is accumulator slot n % 16 of block
// n / 16; its weight P = 2^(c s - mc) (mc = c m) is rounded to bf16 and paired
// with its neighbour: pair i = n / 2 is dword i % 4 of the P^T operand p[i / 4]
// (low half: the even score).  The lane sum adds exactly these bf16 values.
// In the pipelined loop it runs on the matrix cores: v_mfma_f32_4x4x4bf16_1k
// with A = ones returns in every lane the fp32 sum of that lane's own four B
// values, so eight of them (two packed pairs each) add up a tile; the vector
// units, which the softmax already loads beyond what the matrix instructions
// hide, are spared the 63 instructions of a VALU sum (v_dot2_f32_bf16 against
// (1, 1) is no better: it stalls the matrix pipe for longer than a 4x4x4 MFMA).
// The unscheduled form below, for the first tile and the rare path, reads the
// pair back instead -- the high half as a float is (bits & 0xffff0000), the low
// half (bits << 16) -- and adds in fp32.
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }

__device__ __forceinline__ void store_pairs(const uint32_t (&w)[16], bf16x8_t (&p)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]});
}

// All 32 weights of a tile and their lane sum (the unscheduled form, for the
// first tile and the rare path).
__device__ __forceinline__ float weights(const f32x16_t (&s)[2], float c, float mc, bf16x8_t (&p)[4]) {
  uint32_t w[16];
  float hi = 0.f, lo = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kb = i >> 3, e = 2 * (i & 7);
    w[i] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[kb][e], c, -mc)),
                       __builtin_amdgcn_exp2f(fmaf(s[kb][e + 1], c, -mc)));
    hi += hi_bf16(w[i]);
    lo += lo_bf16(w[i]);
  }
  store_pairs(w, p);
  return hi + lo;
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
  return weights(s, c, m_new * c, p);
}

// Rare path of the log2 variant, where the accumulators hold score - m: move
// m up to the tile's row maximum when that exceeds it, scale O and l, shift the
// next tile's scores (computed against the old m) and the chain start, and
// recompute the tile's weights.
__device__ __forceinline__ float rebase_log2(const f32x16_t (&s_in)[2], f32x16_t (&s_next)[2], State& st,
                                             bf16x8_t (&p)[4]) {
  f32x16_t s[2] = {s_in[0], s_in[1]};
  asm volatile("" : "+v"(s[0]), "+v"(s[1]));
  float m0 = fmaxf(s[0][0], s[0][1]);
  float m1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int e = 2; e < 16; e += 2) {
    m0 = fmaxf(fmaxf(m0, s[0][e]), s[0][e + 1]);
    m1 = fmaxf(fmaxf(m1, s[1][e]), s[1][e + 1]);
  }
  const float delta = fmaxf(pair_max(fmaxf(m0, m1)), 0.f);  // m_new - m_old, same in both halves
  const float alpha = __builtin_amdgcn_exp2f(-delta);
  st.m += delta;
  st.l *= alpha;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.o[i] *= alpha;
  s_next[0] -= delta;
  s_next[1] -= delta;
  st.minit -= delta;
  return weights(s, 1.f, delta, p);
}

// Scores of keys at or past L (only in the last, partial tile) become -inf.
// Accumulator slot 4r + qq of lane half g is tile row 32 kb + 8 r + 4 g + qq,
// which holds key perm(row) in a permuted K tile.
template <bool kPerm>
__device__ __forceinline__ void mask_tail(f32x16_t (&s)[2], int kbase, int L, int g) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int row = 32 * kb + 8 * r + 4 * g + qq;
        if (kbase + (kPerm ? perm(row) : row) >= L) s[kb][4 * r + qq] = -INFINITY;
      }
}

// ---------------------------------------------------------------- kernel
struct Ctx {
  const lds_char* lds;
  uint32_t lds_base;
  const char* kbase;          // K, this head, token 0
  const char* vbase;          // V (row-major: this head, token 0; V^T: this head's first channel row)
  int64_t tile_bytes;         // 64 tokens of K or row-major V
  int64_t row_bytes;          // one token row of all heads
  int64_t vt_valid;           // V^T: bytes from a tile's first byte to its last
  int64_t krow_bytes, ktile_bytes;  // K: one token row, 64 token rows (bf16 or FP8)
  DmaOffsets kdma, vdma;
  int n_full, n_tiles, L, wave, g;
  float c;
};

// DMA of tile t (clamped to the last tile: the refetch past the end keeps the
// number of DMA instructions per iteration fixed) of the tensor at base into
// the LDS buffer at byte offset buf.
__device__ __forceinline__ TileDma dma_tile(const Ctx& x, const char* base, int t, uint32_t buf) {
  t = t < x.n_tiles ? t : x.n_tiles - 1;
  const int64_t valid = (int64_t)(x.L - 1 - t * kBN) * x.row_bytes + kD * 2;
  return tile_dma(base + t * x.tile_bytes, valid, x.lds_base + buf, x.wave);
}
// V^T tile t: 64 keys (128 bytes) of each of the head's 128 channel rows.
__device__ __forceinline__ TileDma dma_vt_tile(const Ctx& x, int t, uint32_t buf) {
  t = t < x.n_tiles ? t : x.n_tiles - 1;
  return tile_dma(x.vbase + t * (kBN * 2), x.vt_valid, x.lds_base + buf, x.wave);
}
template <bool kVT>
__device__ __forceinline__ TileDma dma_v(const Ctx& x, int t, uint32_t buf) {
  return kVT ? dma_vt_tile(x, t, buf) : dma_tile(x, x.vbase, t, buf);
}

// K tile t (clamped to the last tile), bf16 rows or FP8 rows.
template <bool kFp8>
__device__ __forceinline__ TileDma dma_k(const Ctx& x, int t, uint32_t buf) {
  t = t < x.n_tiles ? t : x.n_tiles - 1;
  const int64_t valid = (int64_t)(x.L - 1 - t * kBN) * x.krow_bytes + (kFp8 ? kD : kD * 2);
  return tile_dma(x.kbase + t * x.ktile_bytes, valid, x.lds_base + buf, x.wave);
}
// All of this wave's pieces of a K tile (an FP8 tile has one piece a wave).
template <bool kFp8>
__device__ __forceinline__ void dma_k_all(const TileDma& t, const DmaOffsets& d) {
  if (kFp8) dma_piece(t, d, 0);
  else dma_all(t, d);
}

__device__ __forceinline__ uint32_t ring(int t) { return (uint32_t)(t % kStages) * kTileBytes; }

// The 32 matrix instructions of an iteration, in issue order ("slots"): even
// slot k is score MFMA k/2 (block kb = (k/2) & 1, k-step ks = k/4), odd slot k
// is P*V MFMA (k-1)/2 (16-key step j = k/8, d-block (k/2) & 3).  Chains of
// dependent MFMAs are 4 (scores) or 8 (P*V) slots apart.
template <bool kVT>
__device__ __forceinline__ bf16x8_t slot_operand(int k, const lds_char* lds, const Addr& b) {
  const int i = k >> 1;
  return (k & 1) == 0 ? k_operand(i & 1, i >> 1, lds, b) : v_operand<kVT>(i & 3, i >> 2, lds, b);
}

// Iteration t: S(t+1) from K(t+1) into s_next; O += V(t-1) P(t-1) (skipped for
// t = 0); P(t) from s_cur into p_cur.  K(t+1) sits in ring slot (t+1) % 4 and
// V(t-1) in slot (t-1) % 4.  DMA fills K(t+4) into the K slot of K(t) (read in
// iteration t-1) and V(t+2) into the V slot of V(t-2) (read in iteration t-1);
// the DMA of iteration t-2 (K(t+2), V(t)) must have landed before the barrier
// that ends this one, so each DMA has about two iterations to arrive.  In the
// last iteration there is no K(t+1): S(t+1) is computed from a stale slot and
// never used.
//
// With the P*V product (t > 0) the instruction order is fixed by hand, slot by
// slot, with scheduling barriers in between: the operand read of slot k + 2,
// the MFMA of slot k, then a share of the weights, each step one slot after
// the one it depends on -- the FMA of score k, the exponential of score k - 1,
// on odd slots the bf16 pack of pair (k - 3) / 2, and every fourth slot the
// 4x4x4 MFMA that adds two packed pairs to the row sum.  A slot then holds one
// transcendental and one or two plain VALU instructions next to its 32-cycle
// matrix instruction; four more slots without one finish the last pairs.
// DMA instructions a wave issues per iteration: two pieces of each 16 KiB
// tile, one of an FP8 K tile.
template <bool kFp8>
constexpr int dma_per_iteration() { return (kFp8 ? 1 : kDmaPerWave) + kDmaPerWave; }

template <bool kPV, bool kLog2, bool kVT, bool kFp8>
__device__ __forceinline__ void iteration(const Ctx& x, State& st, Addr& a, const f32x16_t (&s_cur)[2],
                                          f32x16_t (&s_next)[2], const bf16x8_t (&p_prev)[4],
                                          bf16x8_t (&p_cur)[4], int t) {
  static_assert(!kFp8 || (kLog2 && kVT), "the FP8 score product is built on the log2 kernel");
  asm volatile("" : "+v"(a.k), "+v"(a.v0), "+v"(a.v1));
  // The tile descriptors (scalar arithmetic) are made in the slot of their
  // first piece, where the scalar unit works under that slot's matrix
  // instruction, not all at the start of the iteration.
  const auto k_desc = [&]() { return tile_dma(st.kt_base, st.kt_valid, x.lds_base + ring(t), x.wave); };
  const auto v_desc = [&]() {
    return tile_dma(st.vt_base, st.vt_valid, x.lds_base + kVRing + ring(t + kStages - 2), x.wave);
  };
  TileDma kd, vd;
  const Addr b = at_buffers(a, ring(t + 1), kVRing + ring(t + kStages - 1));

  const float c = x.c, mc = st.m * c;
  float psum;
  s_next[0] = kLog2 ? st.minit : f32x16_t{};
  s_next[1] = kLog2 ? st.minit : f32x16_t{};
  if (kFp8 && kPV) {
    // Twenty matrix slots: score MFMA i (k = 64: 32-key block i & 1, k-step
    // i >> 1; twice the issue time of the others) at slot 5 i, P*V MFMA n
    // (d-block n & 3, 16-key step n >> 2) at slot n + n / 4 + 1.  Weights two
    // scores a slot: slot s < 16 exponentiates scores 2s and 2s + 1, slots 1..16
    // pack pair s - 1, and slots 3, 5, .., 17 add pairs s - 3 and s - 2 to the
    // row sum (4x4x4 MFMA).  Operands are read two slots ahead.
    float xs[32];
    uint32_t w[16];
    const i16x4_t ones4 = {16256, 16256, 16256, 16256};  // bf16 1.0
    f32x4_t sum4 = {0.f, 0.f, 0.f, 0.f};
    i32x8_t kop[4];
    bf16x8_t vop[16];
    const auto load_op = [&](int sl) {
      if (sl % 5 == 0) {
        kop[sl / 5] = k8_operand((sl / 5) & 1, (sl / 5) >> 1, x.lds, b);
      } else {
        const int n = sl - sl / 5 - 1;
        vop[n] = v_operand<true>(n & 3, n >> 2, x.lds, b);
      }
    };
    load_op(0);
    load_op(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < 20; ++sl) {
      if (sl == 2) {
        kd = k_desc();
        dma_piece(kd, x.kdma, 0);
      }
      if (sl == 8) {
        vd = v_desc();
        dma_piece(vd, x.vdma, 0);
      }
      if (sl == 14) dma_piece(vd, x.vdma, 1);
      if (sl + 2 < 20) load_op(sl + 2);
      if (sl % 5 == 0) {
        const int i = sl / 5;
        s_next[i & 1] = mfma32_fp8(kop[i], st.q8[i >> 1], s_next[i & 1]);
      } else {
        const int n = sl - sl / 5 - 1;
        st.o[n & 3] = mfma32(vop[n], p_prev[n >> 2], st.o[n & 3]);
      }
      if (sl < 16) {
        xs[2 * sl] = __builtin_amdgcn_exp2f(s_cur[sl >> 3][(2 * sl) & 15]);
        xs[2 * sl + 1] = __builtin_amdgcn_exp2f(s_cur[sl >> 3][(2 * sl + 1) & 15]);
      }
      if (sl >= 1 && sl <= 16) {
        w[sl - 1] = pack_bf16x2(xs[2 * sl - 2], xs[2 * sl - 1]);
        asm volatile("" : "+v"(w[sl - 1]));
      }
      if (sl >= 3 && sl <= 17 && (sl & 1) == 1) {
        const int i = (sl - 3) >> 1;
        const i16x4_t b4 = __builtin_bit_cast(i16x4_t, u32x2_t{w[2 * i], w[2 * i + 1]});
        sum4 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones4, b4, sum4, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_pairs(w, p_cur);
    psum = sum4[0];
  } else if (kPV) {
    float xs[32];
    uint32_t w[16];
    const i16x4_t ones4 = {16256, 16256, 16256, 16256};  // bf16 1.0
    f32x4_t sum4 = {0.f, 0.f, 0.f, 0.f};
    bf16x8_t op[32];
    op[0] = slot_operand<kVT>(0, x.lds, b);
    op[1] = slot_operand<kVT>(1, x.lds, b);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 36; ++k) {
      // This iteration's DMA, one piece every 8 slots: issued all at once by
      // all 8 waves, the loads back up in the address unit and hold the waves
      // at the start of the iteration.
      if (k == 4) {
        kd = k_desc();
        dma_piece(kd, x.kdma, 0);
      }
      if (k == 12) dma_piece(kd, x.kdma, 1);
      if (k == 20) {
        vd = v_desc();
        dma_piece(vd, x.vdma, 0);
      }
      if (k == 28) dma_piece(vd, x.vdma, 1);
      if (k < 32) {
        if (k + 2 < 32) op[k + 2] = slot_operand<kVT>(k + 2, x.lds, b);
        const int i = k >> 1;
        if ((k & 1) == 0) {
          s_next[i & 1] = mfma32(op[k], st.q[i >> 1], s_next[i & 1]);
        } else {
          st.o[i & 3] = mfma32(op[k], p_prev[i >> 2], st.o[i & 3]);
        }
        xs[k] = kLog2 ? s_cur[k >> 4][k & 15] : fmaf(s_cur[k >> 4][k & 15], c, -mc);
      }
      if (k >= 1 && k <= 32) xs[k - 1] = __builtin_amdgcn_exp2f(xs[k - 1]);
      if ((k & 1) == 1 && k >= 3) {
        const int i = (k - 3) >> 1;
        w[i] = pack_bf16x2(xs[2 * i], xs[2 * i + 1]);
        // Opaque: the sums below must read the packed pair, not a second
        // conversion of one of its halves.
        asm volatile("" : "+v"(w[i]));
      }
      if (k >= 6 && ((k - 6) & 3) == 0 && ((k - 6) >> 2) < 8) {
        // Pairs 2i and 2i+1 (packed on slots 4i+3 and 4i+5) into the row sum.
        const int i = (k - 6) >> 2;
        const i16x4_t b4 = __builtin_bit_cast(i16x4_t, u32x2_t{w[2 * i], w[2 * i + 1]});
        sum4 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones4, b4, sum4, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_pairs(w, p_cur);
    psum = sum4[0];
  } else {
    kd = k_desc();
    vd = v_desc();
    dma_k_all<kFp8>(kd, x.kdma);
    dma_all(vd, x.vdma);
    if (kFp8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s_next[kb] = mfma32_fp8(k8_operand(kb, ks, x.lds, b), st.q8[ks], s_next[kb]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s_next[kb] = mfma32(k_operand(kb, ks, x.lds, b), st.q[ks], s_next[kb]);
    }
    psum = kLog2 ? weights(s_cur, 1.f, 0.f, p_cur) : weights(s_cur, c, mc, p_cur);
  }
  // The barrier first: the row-sum test below waits on the last row-sum
  // instruction, and that wait then overlaps the barrier's.  What follows
  // touches registers only.
  dma_wait_all_but<(kStages - 2) * dma_per_iteration<kFp8>()>();  // the last two iterations' DMA may be in flight
  __syncthreads();  // K(t+2), V(t) landed; every wave is done with K(t+1), V(t-1)
  if (__builtin_amdgcn_ballot_w64(!(psum <= kSumBound)) != 0) {
    cold_path();
    psum = kLog2 ? rebase_log2(s_cur, s_next, st, p_cur) : rebase(s_cur, st, c, p_cur);
  }
  st.l += psum;
  if (t + 1 >= x.n_full) {
    cold_path();
    mask_tail<kVT>(s_next, (t + 1) * kBN, x.L, x.g);
  }
  if (t + kStages + 1 < x.n_tiles) {
    st.kt_base += x.ktile_bytes;
    st.kt_valid -= x.ktile_bytes;
  }
  if (t + kStages - 1 < x.n_tiles) {
    st.vt_base += kVT ? kBN * 2 : x.tile_bytes;
    if (!kVT) st.vt_valid -= x.tile_bytes;
  }
}

// A wave none of whose 32 query rows exists (only in the last, partial q-tile
// of a head) still carries its share of the tile DMA and takes part in every
// barrier, so the other waves see the same ring; it computes nothing, which
// leaves its SIMD's matrix core to the wave that shares it.
template <bool kVT, bool kFp8>
__device__ __forceinline__ void stream_only(const Ctx& x) {
  dma_wait();
  __syncthreads();  // the ring fill is in LDS
  __syncthreads();  // the first tile's scores are read
  for (int t = 0; t < x.n_tiles; ++t) {
    dma_k_all<kFp8>(dma_k<kFp8>(x, t + kStages, ring(t)), x.kdma);
    dma_all(dma_v<kVT>(x, t + kStages - 2, kVRing + ring(t + kStages - 2)), x.vdma);
    dma_wait_all_but<(kStages - 2) * dma_per_iteration<kFp8>()>();
    __syncthreads();
  }
  dma_wait();
}

// Q's RMSNorm and MM-RoPE, applied to the raw Q^T operand as it is loaded
// (the Q half of the fused prologue, same RFC, section 5 items
// h3_qk_rmsnorm_d128 and h3_mm_rope_3axis_partial):
//   y_c = x_c (mean(x^2) + 1e-5)^(-1/2) (gamma_c q_scale)
//   out_c = y_c cos phi_c - y_{c+48} sin phi_c, out_{c+48} = y_{c+48} cos phi_c
//   + y_c sin phi_c (c < 48), out_c = y_c (c >= 96), rounded once to bf16.
// Every fp32 operation follows the standalone prologue kernel in value and
// order, so q comes out with the same bits.  That kernel gives a head-row to
// 16 lanes: lane i holds channels 4i..4i+3 and 48+4i..48+4i+3 (i < 12) or
// pass-through channels, and adds its 8 squares in that order.  Those channels
// sit in lane half (i >> 1) & 1 here, so half g holds the 8 lanes
// i = 4m + 2g + o: channels 16m + 8g + 4o.. of q[m] and q[m+3] for m < 3, of
// q[6] and q[7] for m = 3.  Its butterfly (xor 1, 2, 4, 8 over i) is then:
// xor 1 (over o) and xor 4, 8 (over m) inside the lane, xor 2 the exchange
// between the two halves.  IEEE addition commutes, so every partner order
// gives the same sum.  cs_row: the row's cosines (48) then sines (48).
//
// kFp8: the rotated fp32 values, times 4 (exact), are rounded to FP8 e4m3
// instead of bf16 and land in q8: channel 16 ks + 8 g + e (the value q[ks][e]
// would hold) goes to byte 8 (ks % 4) + e of k-step ks / 4 -- the byte order of
// a K8 row's lane half g, so the score product pairs equal channels.
template <bool kFp8>
__device__ __forceinline__ void q_prologue(bf16x8_t (&q)[8], i32x8_t (&q8)[2], int g,
                                           const float* __restrict__ gamma_q, const float* __restrict__ cs_row,
                                           float q_scale) {
  f32x4_t gm[8][2], cs[3][2], sn[3][2];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) gm[ks][h] = *reinterpret_cast<const f32x4_t*>(gamma_q + 16 * ks + 8 * g + 4 * h);
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cs[m][h] = *reinterpret_cast<const f32x4_t*>(cs_row + 16 * m + 8 * g + 4 * h);
      sn[m][h] = *reinterpret_cast<const f32x4_t*>(cs_row + 48 + 16 * m + 8 * g + 4 * h);
    }
  float s[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int ka = m < 3 ? m : 6, kb = m < 3 ? m + 3 : 7;
    float part[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      float ss = (float)q[ka][4 * o] * (float)q[ka][4 * o];
#pragma unroll
      for (int e = 1; e < 4; ++e) ss = fmaf((float)q[ka][4 * o + e], (float)q[ka][4 * o + e], ss);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf((float)q[kb][4 * o + e], (float)q[kb][4 * o + e], ss);
      part[o] = ss;
    }
    s[m] = pair_sum(part[0] + part[1]);
  }
  const float ss = (s[0] + s[1]) + (s[2] + s[3]);
  const float r = 1.0f / sqrtf(ss * (1.0f / kD) + 1e-5f);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int ka = m < 3 ? m : 6, kb = m < 3 ? m + 3 : 7;
    bf16x8_t oa, ob;
    float fa[8], fb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = m < 3 ? cs[m][e >> 2][e & 3] : 1.0f;
      const float sv = m < 3 ? sn[m][e >> 2][e & 3] : 0.0f;
      const float ya = (float)q[ka][e] * r * (gm[ka][e >> 2][e & 3] * q_scale);
      const float yb = (float)q[kb][e] * r * (gm[kb][e >> 2][e & 3] * q_scale);
      fa[e] = fmaf(ya, c, -(yb * sv));
      fb[e] = fmaf(yb, c, ya * sv);
      oa[e] = (__bf16)fa[e];  // round to nearest even
      ob[e] = (__bf16)fb[e];
    }
    if (kFp8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        q8[ka >> 2][2 * (ka & 3) + h] =
            (int)pack_e4m3x4(4.0f * fa[4 * h], 4.0f * fa[4 * h + 1], 4.0f * fa[4 * h + 2], 4.0f * fa[4 * h + 3]);
        q8[kb >> 2][2 * (kb & 3) + h] =
            (int)pack_e4m3x4(4.0f * fb[4 * h], 4.0f * fb[4 * h + 1], 4.0f * fb[4 * h + 2], 4.0f * fb[4 * h + 3]);
      }
    } else {
      q[ka] = oa;
      q[kb] = ob;
    }
  }
}

// kQPro: q holds the raw (pre-prologue) rows and q_prologue is applied at
// the load, with gamma_q, the rope_cs table ([L][96] fp32) and q_scale.
// kFp8 (with the other three): the score product in OCP FP8 e4m3 -- q' times 4
// quantized in the Q prologue, k' / 4 read from the K8 form h3attn_kv_prologue_fp8
// writes (bytes [L][H][128]) -- on v_mfma_scale_f32_32x32x64_f8f6f4 at twice the
// bf16 rate; the softmax, P V and output are those of the log2 variant.
template <bool kLog2, bool kVT, bool kQPro, bool kFp8 = false>
__global__ __launch_bounds__(kThreads, 1) void attention_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, float* __restrict__ lse, int L, int H, int Lp, float scale_log2e, int n_qfull,
    const float* __restrict__ gamma_q, const float* __restrict__ rope_cs, float q_scale, int n_half) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStages * kTileBytes];

  // Blocks are dispatched in increasing order, round-robin over the 8 XCDs
  // (block b -> XCD b % 8).  The first H * n_qfull blocks take the full
  // 256-row q-tiles, renumbered so that each XCD receives a contiguous run of
  // them: the workgroups that share one head's K/V then share one L2.  The
  // last H blocks, dispatched last, take each head's partial q-tile (if L is
  // not a multiple of 256), which finish sooner (see stream_only) and so fill
  // the final round of the grid.  When that round would also hold full
  // q-tiles on otherwise idle CUs, the last n_half full tiles (in head-major
  // order) run instead as two workgroups of 128 rows each, blocks
  // H * n_qfull - n_half .. H * n_qfull + n_half - 1: waves 0..3 own the rows,
  // one per SIMD, and waves 4..7 only stream K/V, so the round ends sooner.  A
  // wave computes its rows the same way in any of these workgroups.
  const int b = blockIdx.x, nfb = H * n_qfull, nwhole = nfb - n_half;
  int head, qtile, row0, active_waves = kWaves;
  if (b < nwhole) {
    const int xcd = b & 7, slot = b >> 3;
    const int per = nwhole >> 3, rem = nwhole & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    head = logical / n_qfull;
    qtile = logical - head * n_qfull;
    row0 = qtile * kBM;
  } else if (b < nfb + n_half) {
    const int j = b - nwhole, logical = nwhole + (j >> 1);
    head = logical / n_qfull;
    qtile = logical - head * n_qfull;
    row0 = qtile * kBM + (j & 1) * (kBM / 2);
    active_waves = kWaves / 2;
  } else {
    head = b - nfb - n_half;
    qtile = n_qfull;
    row0 = qtile * kBM;
  }

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
  x.tile_bytes = (int64_t)kBN * x.row_bytes;
  x.krow_bytes = kFp8 ? tok_stride : x.row_bytes;  // K8: one byte per value
  x.ktile_bytes = (int64_t)kBN * x.krow_bytes;
  x.kbase = reinterpret_cast<const char*>(k) + (int64_t)head * kD * (kFp8 ? 1 : 2);
  x.kdma = kFp8 ? k8_dma_offsets(x.krow_bytes, x.wave, lane) : dma_offsets<kVT>(tok_stride, x.wave, lane);
  if (kVT) {
    const int64_t vt_row_bytes = (int64_t)Lp * 2;  // one channel row of V^T
    x.vbase = reinterpret_cast<const char*>(v + (int64_t)head * kD * Lp);
    x.vt_valid = (kD - 1) * vt_row_bytes + kBN * 2;
    x.vdma = vt_dma_offsets(vt_row_bytes, x.wave, lane);
  } else {
    x.vbase = reinterpret_cast<const char*>(v + (int64_t)head * kD);
    x.vt_valid = 0;
    x.vdma = x.kdma;
  }

  Addr a;
  a.k = kFp8 ? 128u * col + 16u * ((4u * x.g) ^ vswz(col)) : 256u * col + ((16u * x.g) ^ (16u * swz(col)));
  if (kVT) {
    a.v0 = 128u * col + 16u * (x.g ^ vswz(col));  // V^T row col, chunk g (XOR 2j per key step)
    a.v1 = a.v0;
  } else {
    const int key_a = 4 * (lane >> 5) + ((lane & 15) >> 2);  // transposing-read key of this lane
    const int ch = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // transposing-read channel
    a.v0 = 256u * key_a + 8u * ((ch >> 2) & 1) + ((16u * (ch >> 3)) ^ (16u * swz(key_a)));
    a.v1 = 256u * (8 + key_a) + 8u * ((ch >> 2) & 1) + ((16u * (ch >> 3)) ^ (16u * swz(8 + key_a)));
  }

  // Ring fill: K(0) .. K(3), V(0) and V(1).
#pragma unroll
  for (int i = 0; i < kStages; ++i) dma_k_all<kFp8>(dma_k<kFp8>(x, i, ring(i)), x.kdma);
#pragma unroll
  for (int i = 0; i < kStages - 2; ++i) dma_all(dma_v<kVT>(x, i, kVRing + ring(i)), x.vdma);

  if (x.wave >= active_waves || row0 + x.wave * 32 >= L) {
    stream_only<kVT, kFp8>(x);
    return;
  }

  // Q^T operand: lane holds Q[row][16ks + 8g .. +7] for its query row.
  State st;
  const int qrow = row0 + x.wave * 32 + col;
  if (qrow < L) {
    const uint16_t* p = q + (int64_t)qrow * tok_stride + (int64_t)head * kD + 8 * x.g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st.q[ks] = *reinterpret_cast<const bf16x8_t*>(p + 16 * ks);
    if (kQPro) q_prologue<kFp8>(st.q, st.q8, x.g, gamma_q, rope_cs + (int64_t)qrow * 96, q_scale);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st.q[ks] = bf16x8_t{};
    st.q8[0] = st.q8[1] = i32x8_t{};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) st.o[i] = f32x16_t{};
  st.m = -FLT_MAX;
  st.l = 0.f;
  dma_wait();
  __syncthreads();  // the ring fill is in LDS

  f32x16_t s0[2], s1[2];
  bf16x8_t p0[4], p1[4];
  s0[0] = f32x16_t{};
  s0[1] = f32x16_t{};
  {
    const Addr b0 = at_buffers(a, ring(0), kVRing);
    if (kFp8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s0[kb] = mfma32_fp8(k8_operand(kb, ks, x.lds, b0), st.q8[ks], s0[kb]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s0[kb] = mfma32(k_operand(kb, ks, x.lds, b0), st.q[ks], s0[kb]);
    }
  }
  if (x.n_full == 0) mask_tail<kVT>(s0, 0, L, x.g);
  if (kLog2) {
    // The offset starts at the first tile's row maximum, so no tile needs
    // the -FLT_MAX start (which would swamp the scores held relative to m).
    float m0 = fmaxf(s0[0][0], s0[0][1]);
    float m1 = fmaxf(s0[1][0], s0[1][1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) {
      m0 = fmaxf(fmaxf(m0, s0[0][e]), s0[0][e + 1]);
      m1 = fmaxf(fmaxf(m1, s0[1][e]), s0[1][e + 1]);
    }
    st.m = pair_max(fmaxf(m0, m1));
    s0[0] -= st.m;
    s0[1] -= st.m;
#pragma unroll
    for (int i = 0; i < 16; ++i) st.minit[i] = -st.m;
  }
  // The first iteration refills K(0)'s slot with K(3): every wave must be done
  // reading K(0) first.  (Later refills are ordered by the previous
  // iteration's barrier.)
  __syncthreads();

  // S(t) and P(t) live in s/p[t % 2]; odd/even pairs keep that choice static.
  {
    const int kt = kStages < x.n_tiles ? kStages : x.n_tiles - 1;
    st.kt_base = x.kbase + kt * x.ktile_bytes;
    st.kt_valid = (int64_t)(x.L - 1 - kt * kBN) * x.krow_bytes + (kFp8 ? kD : kD * 2);
    const int vt = kStages - 2 < x.n_tiles ? kStages - 2 : x.n_tiles - 1;
    st.vt_base = x.vbase + (kVT ? (int64_t)vt * kBN * 2 : vt * x.tile_bytes);
    st.vt_valid = kVT ? x.vt_valid : (int64_t)(x.L - 1 - vt * kBN) * x.row_bytes + kD * 2;
  }
  iteration<false, kLog2, kVT, kFp8>(x, st, a, s0, s1, p1, p0, 0);
  int t = 1;
  for (; t + 1 < x.n_tiles; t += 2) {
    iteration<true, kLog2, kVT, kFp8>(x, st, a, s1, s0, p0, p1, t);
    iteration<true, kLog2, kVT, kFp8>(x, st, a, s0, s1, p1, p0, t + 1);
  }
  // P(n-1) V(n-1); V(n-1) landed before the last iteration's barrier.
  const Addr b_last = at_buffers(a, 0, kVRing + ring(x.n_tiles - 1));
  if (t < x.n_tiles) {
    iteration<true, kLog2, kVT, kFp8>(x, st, a, s1, s0, p0, p1, t);
    pv<kVT>(st, p1, x.lds, b_last);
  } else {
    pv<kVT>(st, p0, x.lds, b_last);
  }
  dma_wait();  // the refetches past the end, before the workgroup exits

  // Epilogue: full row sum = both lane-halves; O / l -> bf16.  With lse, the
  // row's natural log-sum-exp of the scaled scores, ln 2 * log2(sum_j 2^(c s_j))
  // = ln 2 * (c m + log2 l) (log2 variant: m + log2 l), for the backward pass.
  const float l_row = pair_sum(st.l);
  const float inv_l = 1.0f / l_row;
  if (lse != nullptr && x.g == 0 && qrow < L)
    lse[(int64_t)head * L + qrow] = kLn2 * ((kLog2 ? st.m : st.m * x.c) + log2f(l_row));
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

// Compute units of the current device (the launch's round size), looked up
// once per device; 256 (MI355X) if the query fails.
static int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// How many of the last full q-tiles run as two 128-row workgroups.  With one
// workgroup per CU, the grid runs in rounds of `cus` workgroups; when its last
// round holds full tiles and there is room to run each of them as two half
// tiles, it does (the half tiles finish sooner: one wave per SIMD, half the
// rows); otherwise none.  The result bits do not depend on this choice.
int forward_half_tiles(int64_t L, int32_t H) {
  const int64_t nfull = (L / kBM) * H, npart = (L % kBM) ? H : 0;
  const int64_t cus = device_cu_count();
  const int64_t last = (nfull + npart) % cus;  // workgroups in the last round
  const int64_t flast = last - npart;          // the full tiles among them
  if (last == 0 || flast <= 0 || last + flast > cus || flast > 1024) return 0;
  return (int)flast;
}

// Workgroups of a forward launch: every q-tile, plus one per tile run as two
// halves; the bound attention_grid_blocks (used by validation, which makes no
// HIP call) allows for up to 1024 of those.
static dim3 forward_grid(int64_t L, int32_t H, int n_half) {
  return dim3((unsigned)(((L + kBM - 1) / kBM) * (int64_t)H + n_half));
}
int64_t attention_grid_blocks(int64_t L, int32_t H) {
  const int64_t nfull = (L / kBM) * H;
  return ((L + kBM - 1) / kBM) * (int64_t)H + (nfull < 1024 ? nfull : 1024);
}
int attention_block_threads() { return kThreads; }

// One past the last byte, counted from the tile's first byte, that a tile DMA
// reads (dma_offsets: row kBN - 1, chunk 15; vt_dma_offsets: channel row
// kD - 1, chunk 7).  The per-lane offsets are 32-bit and the buffer size is
// clamped to 2^32 - 1, so a geometry whose end exceeds that would wrap.
int64_t row_tile_dma_end(int32_t H) { return (int64_t)(kBN - 1) * H * kD * 2 + kD * 2; }
int64_t vt_tile_dma_end(int64_t L) { return (int64_t)(kD - 1) * vt_padded_length(L) * 2 + kBN * 2; }

int64_t vt_padded_length(int64_t L) { return (L + kBN - 1) / kBN * kBN; }
int64_t vt_bytes(int64_t L, int32_t H) { return (int64_t)H * kD * vt_padded_length(L) * 2; }
hipError_t launch_attention_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    uint16_t* out, float* lse, int64_t L, int32_t H, float scale, bool log2,
                                    hipStream_t stream) {
  const int n_qfull = (int)(L / kBM);  // full 256-row q-tiles per head
  const int n_half = forward_half_tiles(L, H);
  const dim3 grid = forward_grid(L, H, n_half);
  if (log2)  // v is V^T
    hipLaunchKernelGGL((attention_fwd_kernel<true, true, false>), grid, dim3(kThreads), 0, stream, q, k, v, out,
                       lse, (int)L, (int)H, (int)vt_padded_length(L), 1.0f, n_qfull, nullptr, nullptr, 1.0f, n_half);
  else
    hipLaunchKernelGGL((attention_fwd_kernel<false, false, false>), grid, dim3(kThreads), 0, stream, q, k, v, out,
                       lse, (int)L, (int)H, 0, scale * kLog2e, n_qfull, nullptr, nullptr, 1.0f, n_half);
  return hipGetLastError();
}

hipError_t launch_attention_forward_fp8(const uint16_t* q_raw, const uint8_t* k8, const uint16_t* vt, uint16_t* out,
                                        const float* gamma_q, const float* rope_cs, int64_t L, int32_t H,
                                        float q_scale, hipStream_t stream) {
  const int n_qfull = (int)(L / kBM);
  const int n_half = forward_half_tiles(L, H);
  hipLaunchKernelGGL((attention_fwd_kernel<true, true, true, true>), forward_grid(L, H, n_half), dim3(kThreads), 0,
                     stream, q_raw, reinterpret_cast<const uint16_t*>(k8), vt, out, nullptr, (int)L, (int)H,
                     (int)vt_padded_length(L), 1.0f, n_qfull, gamma_q, rope_cs, q_scale, n_half);
  return hipGetLastError();
}

hipError_t launch_attention_forward_qprologue(const uint16_t* q_raw, const uint16_t* k, const uint16_t* vt,
                                              uint16_t* out, const float* gamma_q, const float* rope_cs,
                                              int64_t L, int32_t H, float q_scale, hipStream_t stream) {
  const int n_qfull = (int)(L / kBM);
  const int n_half = forward_half_tiles(L, H);
  hipLaunchKernelGGL((attention_fwd_kernel<true, true, true>), forward_grid(L, H, n_half), dim3(kThreads), 0, stream,
                     q_raw, k, vt, out, nullptr, (int)L, (int)H, (int)vt_padded_length(L), 1.0f, n_qfull, gamma_q,
                     rope_cs, q_scale, n_half);
  return hipGetLastError();
}

}  // namespace h3attn
