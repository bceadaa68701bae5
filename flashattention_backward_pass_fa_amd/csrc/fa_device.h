// fa_device.h - device-side helpers shared by the gfx950 kernels.
//
// MFMA operand layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + s], s = 0..7
//                             B (16 x 32): lane l holds B[8 * (l / 32) + s][l % 32]
//                             C (32 x 32): lane l, register r holds
//                                          C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// The accumulator of one product therefore has the *column* index across
// lanes and the row index inside the lane, which is exactly the A/B operand
// shape "row across lanes, reduction index inside the lane" of a product
// that reduces over the first product's rows.  Such register-to-operand
// reuse sees the reduction index in the permuted order
//   k-step u, slot s, lane half g  ->  row 16 u + 8 (s / 4) + 4 g + s % 4,
// and the other operand is then read from LDS in that same order.
//
// ds_read_tr16_b64 (gfx950): within each group of 16 lanes, lane i, slot s
// receives element i % 4 of the 8-byte chunk addressed by lane 4 s + i / 4.
// If lane j of the group addresses row R + j / 4, column C + 4 (j % 4) of a
// row-major bf16 tile, lane i receives rows R..R+3 of column C + i: a
// k-inside-lane operand read straight from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Element type of the 16-bit MFMA kernels.  Their sources (fa_fwd16.hip,
// fa_bwd16.hip) are compiled twice: for bf16, and with FA_ELEM_F16 for fp16,
// whose kernels and launchers live in namespace fa::fp16.
#ifdef FA_ELEM_F16
typedef f16 e16;
typedef f16x8 e16x8;
typedef f16x4 e16x4;
#define FA_ELEM_NS_BEGIN namespace fp16 {
#define FA_ELEM_NS_END }
#define FA_ELEM_NS fp16::
#else
typedef bf16 e16;
typedef bf16x8 e16x8;
typedef bf16x4 e16x4;
#define FA_ELEM_NS_BEGIN
#define FA_ELEM_NS_END
#define FA_ELEM_NS
#endif
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

// Strided view of one [B, H, N, d] tensor (element strides; d-stride 1).
struct TensorView {
  void* ptr;
  int64_t sb, sh, sn;
};

// Mask, sequence and dropout flags of one call, in the form the kernels use.
// Query i of a sequence with nq queries and nk keys stands at key position
// i + nk - nq (the last query aligns with the last key), so causal hides
// j > i + nk - nq; that shift, causality and the window are folded into two
// offsets.  The host fills the call-wide values (nq, nk = the longest
// sequences); seq_localize turns them into those of one sequence.
struct MaskArgs {
  int nq, nk;         // query and key rows of the sequence
  int causal;         // causal mask requested (used only to order work)
  int lo_off, hi_off; // visible iff i - lo_off <= j <= i + hi_off
  const int* cu_q;    // varlen: sequence b has rows [cu_q[b], cu_q[b+1]) of the packed
  const int* cu_k;    //   query tensors and [cu_k[b], cu_k[b+1]) of the key ones; else null
  int dropout;        // 0/1
  uint32_t keep_threshold;  // keep iff the 16-bit Philox draw >= threshold
  float keep_scale;         // 1 / (1 - p)
  uint32_t seed_lo, seed_hi, off_lo, off_hi;
};

// First packed row of one sequence's queries and keys.
struct SeqRows {
  int q0, k0;
};

// Specialise the call-wide mask to sequence b: its lengths (varlen: from the
// offset arrays, clamped to [0, longest]) and the bottom-right shift
// nk - nq folded into the offsets.  Returns the sequence's first rows.
__device__ __forceinline__ SeqRows seq_localize(MaskArgs& m, int b) {
  SeqRows r{0, 0};
  if (m.cu_q) {
    r.q0 = m.cu_q[b];
    r.k0 = m.cu_k[b];
    m.nq = min(max(m.cu_q[b + 1] - r.q0, 0), m.nq);
    m.nk = min(max(m.cu_k[b + 1] - r.k0, 0), m.nk);
  }
  const int shift = m.nk - m.nq;
  m.lo_off -= shift;
  m.hi_off += shift;
  return r;
}

// Move a tensor view to the first packed row of a sequence (varlen; the
// host zeroes the batch stride there).
template <typename T>
__device__ __forceinline__ void shift_rows(TensorView& t, int rows) {
  t.ptr = (T*)t.ptr + (int64_t)rows * t.sn;
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 8 bytes (4 16-bit elements) transposed out of LDS, see the header comment.
__device__ __forceinline__ e16x4 lds_read_tr(const e16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p));
  return __builtin_bit_cast(e16x4, v);
}

__device__ __forceinline__ e16x8 concat(e16x4 lo, e16x4 hi) {
  return e16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// k-inside-lane operand for one 32x32x16 step from a row-major 16-bit tile
// (row stride ld elements): lane l gets rows row_lo + (0..3) and
// row_hi + (0..3) of column col0 + l % 32, where row_lo/row_hi already
// include the lane half's offset.  Every lane passes its own row bases.
__device__ __forceinline__ e16x8 tr_operand(const e16* tile, int ld, int row_lo, int row_hi,
                                            int col0, int lane) {
  const int j = lane & 15;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const e16x4 lo = lds_read_tr(tile + (row_lo + (j >> 2)) * ld + col);
  const e16x4 hi = lds_read_tr(tile + (row_hi + (j >> 2)) * ld + col);
  return concat(lo, hi);
}

// Row stride (16-bit elements) of a row-major LDS tile of `cols` columns.
// Measured on gfx950 (64 banks of 4 bytes): a b128 row read by 16 lanes of
// consecutive rows is conflict-free when the stride in dwords is an odd
// multiple of 4 modulo 64, and the transposed 8-byte read, which touches 4
// consecutive rows x 8 dwords per 16 lanes, needs those 4 row segments on
// disjoint banks.  76 dwords (128 columns) and 52 dwords (64 columns)
// satisfy both.
__host__ __device__ constexpr int lds_stride(int cols) { return cols == 128 ? 152 : 104; }

// valid(i, j): key j visible to query i ("Lecture 7", "Mask behaviour").
// Causal, window and alignment bounds are folded into two offsets, so the
// test is branch-free.
__device__ __forceinline__ bool visible(const MaskArgs& m, int i, int j) {
  return (i < m.nq) & (j < m.nk) & (j >= i - m.lo_off) & (j <= i + m.hi_off);
}

// Barrier that orders LDS accesses only: global stores and atomics in flight
// are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Philox4x32-10 (Salmon et al., SC'11): the four output words of the block
// for counter (c0, c1, c2, c3) under key (k0, k1).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32 -> 64-bit product per multiplier (a single v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)M0 * c0;
    const uint64_t p1 = (uint64_t)M1 * c2;
    // a ^ b ^ c as one gfx950 three-input bitwise instruction (truth
    // table 0x96); the compiler emits two XORs for the plain expression
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += W0;
    k1 += W1;
  }
  return u32x4{c0, c1, c2, c3};
}

// Dropout keep bits of one Philox block of row i of head (b, h): the block
// at j0 (j0 % 16 = 0 or 4) serves keys j0 .. j0 + 3 and j0 + 8 .. j0 + 11
// (positions 0 .. 7), counter (off_lo, off_hi, (i << 16) | j0,
// (b << 16) | h); position q draws the 16-bit half q % 2 (low first) of
// word q / 2 and is kept iff that draw >= threshold (ceil(p 2^16)).  Bit q
// of the result is position q.  (Runs of four keys eight apart are what
// one lane holds of a 32-key tile in the MFMA accumulator layout.)
__device__ __forceinline__ uint32_t dropout_keep8(const MaskArgs& m, int b, int h, int i, int j0) {
  const u32x4 x = philox4x32_10(m.off_lo, m.off_hi, ((uint32_t)i << 16) | (uint32_t)j0,
                                ((uint32_t)b << 16) | (uint32_t)h, m.seed_lo, m.seed_hi);
  const uint32_t t = m.keep_threshold;
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    r |= ((uint32_t)((x[w] & 0xFFFFu) >= t) << (2 * w)) | ((uint32_t)((x[w] >> 16) >= t) << (2 * w + 1));
  return r;
}

// Keep bit of one element (i, j).
__device__ __forceinline__ bool dropout_keep(const MaskArgs& m, int b, int h, int i, int j) {
  const int j0 = (j & ~15) | (j & 4), q = ((j >> 1) & 4) | (j & 3);
  return (dropout_keep8(m, b, h, i, j0) >> q) & 1u;
}

// Keep bits of this lane's keys of a 32-key tile (j0 % 32 = 0) of row i
// when the lane holds keys j0 + 8 rr + 4 g + (0..3), rr = 0..3 (lane half
// g): exactly the two blocks at j0 + 4 g and j0 + 16 + 4 g.  Bit 4 rr + e
// is key j0 + 8 rr + 4 g + e.
__device__ __forceinline__ uint32_t dropout_keep_lane(const MaskArgs& m, int b, int h, int i, int j0,
                                                      int g) {
  return dropout_keep8(m, b, h, i, j0 + 4 * g) | (dropout_keep8(m, b, h, i, j0 + 16 + 4 * g) << 8);
}

// The same eight keep decisions as dropout_keep8 (position q: half q % 2
// of word q / 2 against the threshold), laid out for the key-octet trade:
// position q at bit (q / 2) + 4 (q % 2).  Both halves of a word are tested
// by two packed 16-bit instructions: a saturating subtraction of
// threshold - 1 leaves a half nonzero iff it is >= threshold (threshold >= 1
// whenever dropout is on), and a minimum with 1 turns that into bits 0 and
// 16.  (Written as instructions: the compiler turns the same expression
// into two compares and two selects per word.)
__device__ __forceinline__ uint32_t dropout_keep8_split(const MaskArgs& m, int b, int h, int i, int j0) {
  const u32x4 x = philox4x32_10(m.off_lo, m.off_hi, ((uint32_t)i << 16) | (uint32_t)j0,
                                ((uint32_t)b << 16) | (uint32_t)h, m.seed_lo, m.seed_hi);
  const uint32_t tm1 = (m.keep_threshold - 1u) & 0xFFFFu;
  const uint32_t t2 = tm1 | (tm1 << 16), ones = 0x00010001u;
  uint32_t v = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t xw = x[w];
    uint32_t y;
    asm("v_pk_sub_u16 %0, %1, %2 clamp\n\tv_pk_min_u16 %0, %0, %3" : "=&v"(y) : "v"(xw), "s"(t2), "s"(ones));
    v |= y << w;
  }
  return (v | (v >> 12)) & 0xFFu;
}

// Word e of a key octet's trade (dropout_keep_octet): QP broadcasts quad
// lane e's draws to its quad; a rotation by eight lanes (DPP row_ror:8) of
// that brings the other quad's lane e.  The quad with key bit 3 clear drew
// rr = 0, 1, the other rr = 2, 3; byte rr of the result is row rr's block.
template <int QP>
__device__ __forceinline__ uint32_t octet_trade(uint32_t mine, int hq) {
  const uint32_t own = (uint32_t)__builtin_amdgcn_mov_dpp((int)mine, QP, 0xF, 0xF, false);
  const uint32_t oth = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0x128, 0xF, 0xF, false);
  return hq ? (oth | (own << 16)) : (own | (oth << 16));
}

// Keep bits of a 32-query x 32-key tile whose keys lie across lanes (this
// lane: key `key`, lane half g) and whose rows q0 + 8 rr + 4 g + e lie
// inside the lane.  The eight lanes of a block (two quads eight lanes
// apart) share each row's Philox block: the lane with key bit 3 = hq and
// key % 4 = e draws rows rr = 2 hq and 2 hq + 1, and the eight trade them.
// Bit 8 rr + dropout_octet_bit(key) of kq[e] is the keep bit of row
// q0 + 8 rr + 4 g + e.  Every lane of the wave must call it.
__device__ __forceinline__ void dropout_keep_octet(const MaskArgs& m, int b, int h, int q0, int g,
                                                   int key, uint32_t (&kq)[4]) {
  const int hq = (key >> 3) & 1, j0 = (key & ~15) | (key & 4);
  const int row = q0 + 16 * hq + 4 * g + (key & 3);  // rr = 2 hq
  const uint32_t mine = dropout_keep8_split(m, b, h, row, j0) | (dropout_keep8_split(m, b, h, row + 8, j0) << 8);
  kq[0] = octet_trade<0x00>(mine, hq);  // quad_perm [0,0,0,0]
  kq[1] = octet_trade<0x55>(mine, hq);  // quad_perm [1,1,1,1]
  kq[2] = octet_trade<0xAA>(mine, hq);  // quad_perm [2,2,2,2]
  kq[3] = octet_trade<0xFF>(mine, hq);  // quad_perm [3,3,3,3]
}

// All ones if bit `pos` of `bits` is set, else zero (a signed one-bit field
// extract), and a float kept or zeroed by such a mask (+0 when zeroed, as a
// select would give).
__device__ __forceinline__ uint32_t bit_mask(uint32_t bits, int pos) {
  return (uint32_t)__builtin_amdgcn_sbfe((int)bits, pos, 1);
}
__device__ __forceinline__ float masked(float v, uint32_t m) { return __uint_as_float(__float_as_uint(v) & m); }

// Position of key `key` in its Philox block (bit index in dropout_keep8).
__device__ __forceinline__ int dropout_pos(int key) { return ((key >> 1) & 4) | (key & 3); }

// Bit of key `key` inside a byte of dropout_keep_octet's words (the
// position's bit in dropout_keep8_split).
__device__ __forceinline__ int dropout_octet_bit(int key) {
  const int q = dropout_pos(key);
  return (q >> 1) + 4 * (q & 1);
}

// Address of row `row` (0 <= row < 2^31) of one head whose rows are `rs`
// bytes apart (rs < 2^32): a single 32 x 32 -> 64-bit multiply-add.
__device__ __forceinline__ const char* row_addr(const char* head, uint32_t rs, int row) {
  return head + (uint64_t)(uint32_t)row * rs;
}

// Head (bh) and block (blk) of this workgroup, for a grid of (heads,
// blocks).  The hardware deals workgroup L (linear launch index) to XCD
// L % 8 and, inside an XCD, hands consecutive workgroups to its shader
// arrays in turn (measured: with a grid x extent that is a multiple of 32,
// every workgroup of a head lands on one array).  The plain mapping (x =
// head, y = block) keeps a head on one XCD (its K, V, Q, dO share that
// XCD's L2) and gives each array whole heads: right when all heads carry the
// same work.  Packed variable-length batches (varlen) do not: a long
// sequence's heads would sit on one array while the others idle on short
// ones.  There, with the head count a multiple of 8 and the block count of 4
// (the launchers pad it), L is re-read so that a head still stays on one
// XCD but each run of four consecutive workgroups of an XCD is four
// consecutive blocks of one head, one per array, snaking (every other run
// backwards, which evens out work that falls linearly with the block), and
// block-major across heads so the longest blocks still start first.
__device__ __forceinline__ void wg_coords(bool varlen, int& bh, int& blk) {
  const int nh = gridDim.x, nb = gridDim.y;
  if (varlen && (nh & 7) == 0 && (nb & 3) == 0) {
    const int L = blockIdx.y * nh + blockIdx.x;
    const int k = L >> 3, run = k >> 2, per_xcd = nh >> 3;
    const int blk4 = run / per_xcd, t = k & 3;
    bh = (L & 7) + 8 * (run % per_xcd);
    blk = 4 * blk4 + ((blk4 & 1) ? 3 - t : t);
  } else {
    bh = blockIdx.x;
    blk = blockIdx.y;
  }
}

// Block count of a grid over n rows in tiles of `tile` (padded to a multiple
// of 4 for wg_coords' varlen mapping).
__host__ __device__ constexpr int grid_blocks(int heads, int n, int tile, bool varlen) {
  return varlen && heads % 8 == 0 ? ((n + tile - 1) / tile + 3) / 4 * 4 : (n + tile - 1) / tile;
}

template <typename T>
__device__ __forceinline__ T* at(const TensorView& t, int b, int h, int n) {
  return (T*)t.ptr + (int64_t)b * t.sb + (int64_t)h * t.sh + (int64_t)n * t.sn;
}


}  // namespace fa
