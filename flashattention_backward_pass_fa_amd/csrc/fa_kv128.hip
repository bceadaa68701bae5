// fa_kv128.hip - the KV-outer backward kernel for head dimension 128
// (deterministic mode), 16-bit (bf16 or fp16): compiled once per element type
// like fa_bwd16.hip, and with the instruction-level-parallelism scheduler.

#include <type_traits>

#include "fa_bwd_common.h"

namespace fa {
FA_ELEM_NS_BEGIN
namespace {

// --------------------------------- KV-outer, d = 128: two phases per block

// P~ (the kept weights, without 1 / (1 - p)) and dS of one 32-key x 32-query
// tile from its S = Q K^T and dP = dO V^T accumulators (keys across lanes,
// queries inside the lane: element r of lane l is query q0 + 8 (r / 4) +
// 4 g + r % 4, key `key`).  MASK zeroes hidden pairs; DROP applies the keep
// mask, one Philox block per eight keys shared by the eight lanes holding them.
// sDq holds -D.  Returns the values as four runs of 4 consecutive queries
// (rr = 0..3).
template <bool MASK, bool DROP>
__device__ __forceinline__ void kv_p_ds(const BwdArgs& a, const f32x16& s, const f32x16& dp,
                                        const float* sLq, const float* sDq, int g, int b, int h,
                                        int q0, int key, e16x4 (&pw)[4], e16x4 (&dw)[4]) {
  uint32_t kq[4] = {~0u, ~0u, ~0u, ~0u};
  const int t = dropout_octet_bit(key);
  if (DROP) dropout_keep_octet(a.m, b, h, q0, g, key, kq);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const f32x4 l4 = *(const f32x4*)(sLq + 8 * rr + 4 * g);
    const f32x4 nd4 = *(const f32x4*)(sDq + 8 * rr + 4 * g);  // -D
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * rr + e;
      float p = fast_exp2(s[r] * a.scale_log2 - l4[e]);
      if (MASK) p = visible(a.m, q0 + 8 * rr + 4 * g + e, key) ? p : 0.f;
      const float dpv = dp[r];
      if (DROP) {
        // dS (1 - p) = P~ dP - P D (1 - p): 1 / (1 - p) is applied to dV and
        // dK at the store, and nd4 holds -D (1 - p)
        const float pk = masked(p, bit_mask(kq[e], 8 * rr + t));
        pw[rr][e] = (e16)pk;
        dw[rr][e] = (e16)fmaf(pk, dpv, p * nd4[e]);
      } else {
        pw[rr][e] = (e16)p;
        dw[rr][e] = (e16)(p * (dpv + nd4[e]));
      }
    }
  }
}

// KV-outer kernel for d = 128 with 8 waves, split into producers and
// consumers ("FlashAttention backward", "The loop structure": dK and dV of
// a key block accumulate in registers over the query blocks and are written
// once).  One workgroup owns 128 keys and loops over the 64-query blocks that
// can see them; in the iteration for block i:
//  - producer wave p (waves 0..3) takes key group p (32 keys, K and V in
//    registers) and all 64 queries of block i + 1: S = Q K^T and dP = dO V^T
//    on MFMA, then P~ and dS ("Lecture 7", "The recomputation trick";
//    "FlashAttention backward", "The gradients, and the one scalar that
//    makes them local"), written key-major (16-bit) to one of two LDS
//    buffers;
//  - consumer wave c (waves 4..7) owns columns 32 c .. 32 c + 31 of dV and dK
//    for all 128 keys and accumulates block i from the other buffer:
//    dV += P~^T dO and dK += dS^T Q in fp32 registers.
// Each SIMD runs one producer and one consumer, so the producers'
// exponentials overlap the consumers' products; the consumers read each Q,
// dO tile once (transposed, for their column slice) instead of once per key
// group, and every dK, dV value has a single owner (no partial sums).
template <int D>
struct KvSCfg {
  static constexpr int BC = 128, BR = 64, NT = 512;
  // P~ and dS tiles, [key][query]: 72 elements = 36 dwords per row, an odd
  // multiple of 4 modulo 64, so the 16-byte A-operand reads of 16 lanes
  // (16 consecutive keys) fall on disjoint banks
  static constexpr int LDP = BR + 8;
  static constexpr int KT = D / 16;
  static constexpr int TILE = BR * D;  // one unpadded Q or dO tile (16 KB)
  // 1 KB LDS-DMA pieces of a Q, dO tile pair per consumer wave
  static constexpr int PIECES = 2 * TILE * 2 / 1024 / 4;
};

// Q and dO tiles are stored unpadded (LDS-DMA writes whole 1 KB pieces, so
// rows cannot be padded) with 16-byte chunk k of row r in slot
// k ^ tile_swz(r) of that row.  The swizzle, a bijection on r % 16, keeps
// both reads conflict-free on gfx950's 64 banks: 16 lanes reading one chunk
// of 16 consecutive rows, and the transposed 8-byte reads of 4 consecutive
// rows x 4 consecutive chunks.
__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// One 16-byte-per-lane LDS-DMA: lane l's 16 bytes at src land at LDS byte
// address lds + 16 l (lds wave-uniform).  Written as assembly so that the
// compiler, which cannot tell these LDS writes from later LDS reads, does
// not wait for the request before every one of them; the issuing wave
// waits (vmcnt) before the barrier that publishes the data.  The request
// has no register result, and the compiler's own vmcnt waits stay correct
// (an extra outstanding request only makes them wait longer).  No code in
// this file uses M0 otherwise; one wait state is needed between writing M0
// and the request.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int D, bool DROP>
__device__ __forceinline__ void dkdv_ws_body(BwdArgs& a, int bh, int blk) {
  static_assert(D == 128, "four 32-column slices per matrix: one per consumer wave");
  using C = KvSCfg<D>;
  constexpr int TILE = C::TILE, PT = C::BC * C::LDP;
  // [0, 4 TILE): Q, dO tiles of two blocks (Q then dO per block); then two
  // P~ / dS buffer pairs; all of it reused for staging the output rows after
  // the loop
  __shared__ __attribute__((aligned(16))) e16 smem[4 * TILE + 4 * PT];
  __shared__ __attribute__((aligned(16))) float sL[2][C::BR];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BR];
  auto sQ = [&](int buf) { return smem + 2 * buf * TILE; };
  auto sO = [&](int buf) { return smem + (2 * buf + 1) * TILE; };
  auto sP = [&](int buf) { return smem + 4 * TILE + 2 * buf * PT; };
  auto sS = [&](int buf) { return smem + 4 * TILE + (2 * buf + 1) * PT; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, as a scalar
  const bool producer = wu < 4;
  const int role = wu & 3;  // producer: key group; consumer: column slice
  const int b = bh / a.H, h = bh - b * a.H;
  bwd_localize(a, b);
  const int NQ = a.m.nq, NK = a.m.nk;
  const int kv0 = blk * C::BC;
  if (kv0 >= NK) return;  // past this sequence's keys
  const int kvw = kv0 + 32 * role;
  const int key = kvw + c;

  // Query rows that can see at least one of the block's keys.
  const int q_lo = max(0, kv0 - a.m.hi_off), q_hi = min(NQ, kv0 + C::BC + a.m.lo_off);
  const int it0 = q_lo / C::BR;
  const int it1 = q_lo < q_hi ? (q_hi + C::BR - 1) / C::BR : it0;

  const int64_t row_base = (int64_t)bh * a.ln;
  const char* q_head = (const char*)at<e16>(a.q, b, h, 0);
  const char* o_head = (const char*)at<e16>(a.dout, b, h, 0);
  const uint32_t q_rs = (uint32_t)a.q.sn * 2, o_rs = (uint32_t)a.dout.sn * 2;
  // Block it's Q and dO rows into tile buffer buf by LDS-DMA (consumer
  // waves): consumer `role` moves PIECES 1 KB pieces of four rows (pieces
  // 0..15: Q, 16..31: dO); lane l of a piece fetches, for row 4 p + l / 16,
  // the chunk that belongs in slot l % 16.  Rows past the end read the last
  // row (finite; every use of them is masked or never stored).
  auto dma_tile = [&](int it, int buf) {
#pragma unroll
    for (int x = 0; x < C::PIECES; ++x) {
      const int piece = C::PIECES * role + x;
      const int mat = piece >> 4, grp = piece & 15;
      const int row = 4 * grp + (lane >> 4);
      const int chunk = (lane & 15) ^ tile_swz(row);
      const char* src = row_addr(mat ? o_head : q_head, mat ? o_rs : q_rs, min(it * C::BR + row, NQ - 1)) + 16 * chunk;
      lds_dma16(src, __builtin_amdgcn_readfirstlane(lds_address(smem + (2 * buf + mat) * TILE + 512 * grp)));
    }
  };
  // L (as L log2 e) and -D of one block, moved by waves 0 and 1
  float pld = 0.f;
  auto ld_load = [&](int it) {
    if (tid < 2 * C::BR)
      pld = (tid < C::BR ? a.lse : a.delta)[row_base + min(it * C::BR + (tid & (C::BR - 1)), NQ - 1)];
  };
  auto ld_store = [&](int buf) {
    if (tid < C::BR) sL[buf][tid] = pld * kLog2e;
    else if (tid < 2 * C::BR) sD[buf][tid - C::BR] = -pld / a.m.keep_scale;  // -D (1 - p): the start value of dP - D without dropout
  };

  // Query blocks [itA, itB) see all 128 keys with no mask edge: the first
  // query must reach the last key, the last query must still see the first.
  int itA = it1, itB = it1;
  if (kv0 + C::BC <= NK) {
    const int lo = max(0, kv0 + C::BC - 1 - a.m.hi_off);
    const int hi = min(NQ - C::BR, kv0 - C::BR + 1 + a.m.lo_off);
    if (lo <= hi) {
      itA = min(max(it0, (lo + C::BR - 1) / C::BR), it1);
      itB = max(itA, min(it1, hi / C::BR + 1));
    }
  }
  auto is_full = [&](int it) { return it >= itA && it < itB; };
  std::integral_constant<bool, false> general;
  std::integral_constant<bool, true> fast;

  // The two roles run separate copies of the loop (so that neither holds the
  // other's registers) with the same barriers in the same order.  Iteration
  // it: consumers take block it (tile and P~/dS buffer (it - it0) & 1),
  // producers block it + 1 (the other ones).  Block it's tile is dead by then
  // (the producers formed block it, and the consumers read their B operands
  // of it, during the iteration before), so the consumers request block
  // it + 2's Q, dO into it at the top of the iteration and wait for them
  // before its barrier, and waves 0 and 1 store block it + 2's L and D.  The
  // first iteration is preceded by the two first tiles and the producers'
  // pass over block it0.
  if (producer) {
    if (it0 < it1) ld_load(it0);
    // K and V rows: B operands of S and dP, in registers for the whole loop
    e16x8 kreg[C::KT], vreg[C::KT];
    {
      const e16* kp = at<e16>(a.k, b, h, min(key, NK - 1));
      const e16* vp = at<e16>(a.v, b, h, min(key, NK - 1));
#pragma unroll
      for (int t = 0; t < C::KT; ++t) {
        kreg[t] = load8(kp + 16 * t + 8 * g);
        vreg[t] = load8(vp + 16 * t + 8 * g);
      }
    }
    if (it0 < it1) ld_store(0);
    // K and V must have landed before the loop: the wait counter cannot tell
    // them from later prefetches, so a register still pending here would
    // make every iteration wait for its own prefetch.
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    lds_barrier();
    // A operand of k-step t: row c of a half, chunk 2 t + g (elements from
    // the half's first row; rows 32 qh + c share c's swizzle)
    int aoff[C::KT];
#pragma unroll
    for (int t = 0; t < C::KT; ++t) aoff[t] = c * D + 8 * ((2 * t + g) ^ tile_swz(c));
    // P~ and dS of block it (both 32-query halves) into buffer pb
    auto produce = [&](int it, int qb, int pb, auto full) {
      constexpr bool FULL = decltype(full)::value;
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const int qs = it * C::BR + 32 * qh;
        e16* prow = sP(pb) + (32 * role + c) * C::LDP + 32 * qh + 4 * g;
        e16* srow = sS(pb) + (32 * role + c) * C::LDP + 32 * qh + 4 * g;
        if (!FULL && block_dead(a.m, qs, 32, kvw, 32)) {
          // a fully hidden tile contributes zeros (the consumers run every
          // tile's products, without branches)
          const e16x4 z4 = {(e16)0.f, (e16)0.f, (e16)0.f, (e16)0.f};
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            *(e16x4*)(prow + 8 * rr) = z4;
            *(e16x4*)(srow + 8 * rr) = z4;
          }
          continue;
        }
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        const e16* qa = sQ(qb) + 32 * qh * D;
#pragma unroll
        for (int t = 0; t < C::KT; ++t) sacc = mfma32x32x16(load8(qa + aoff[t]), kreg[t], sacc);
#pragma unroll
        for (int t = 0; t < C::KT; ++t) dpacc = mfma32x32x16(load8(qa + TILE + aoff[t]), vreg[t], dpacc);
        e16x4 pw[4], dw[4];
        const float* sLq = &sL[qb][32 * qh];
        const float* sDq = &sD[qb][32 * qh];
        if (FULL) kv_p_ds<false, DROP>(a, sacc, dpacc, sLq, sDq, g, b, h, qs, key, pw, dw);
        else kv_p_ds<true, DROP>(a, sacc, dpacc, sLq, sDq, g, b, h, qs, key, pw, dw);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          *(e16x4*)(prow + 8 * rr) = pw[rr];
          *(e16x4*)(srow + 8 * rr) = dw[rr];
        }
      }
    };
    // A block with no mask edge, without dropout, scheduled by hand: the 16
    // products of the second 32-query half are issued among the first
    // half's elementwise work, so that this wave's exponentials run beside
    // its own matrix products instead of after them.  Operands are read
    // AHEAD products early, and dP accumulates from -D, so the product ends
    // as dP - D.  Each step (two products) is fenced so the compiler keeps
    // this order.
    auto produce_full = [&](int it, int qb, int pb) {
      constexpr int AHEAD = 4;
      const e16* qa = sQ(qb);
      // product j: query half j / 16, S = Q K^T (j % 16 < 8) or dP = dO V^T,
      // k-step j % 8
      auto operand = [&](int j) {
        return load8(qa + ((j & 15) < 8 ? 0 : TILE) + (j >> 4) * 32 * D + aoff[j & 7]);
      };
      auto minus_d = [&](int half) {
        f32x16 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x4 d4 = *(const f32x4*)&sD[qb][32 * half + 8 * rr + 4 * g];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * rr + e] = d4[e];
        }
        return v;
      };
      auto log2_l = [&](int half, f32x4 (&l)[4]) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) l[rr] = *(const f32x4*)&sL[qb][32 * half + 8 * rr + 4 * g];
      };
      e16* prow = sP(pb) + (32 * role + c) * C::LDP + 4 * g;
      e16* srow = sS(pb) + (32 * role + c) * C::LDP + 4 * g;
      f32x16 acc[4];  // S, dP - D of half 0, then of half 1
      f32x4 lq[2][4];
      e16x4 pw, dw;
      // P~ = exp2(S scale_log2 - L log2 e) and dS = P~ (dP - D) for
      // elements e, e + 1 of a half; a run of 4 queries is stored when done
      auto pair = [&](int half, int e) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = e + u;
          const float p = fast_exp2(acc[2 * half][r] * a.scale_log2 - lq[half][r >> 2][r & 3]);
          pw[r & 3] = (e16)p;
          dw[r & 3] = (e16)(p * acc[2 * half + 1][r]);
        }
        if ((e & 3) == 2) {
          *(e16x4*)(prow + 32 * half + 8 * (e >> 2)) = pw;
          *(e16x4*)(srow + 32 * half + 8 * (e >> 2)) = dw;
        }
      };
      e16x8 op[AHEAD];
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) op[j] = operand(j);
      acc[0] = f32x16{};
      acc[1] = minus_d(0);
      acc[2] = f32x16{};
      log2_l(0, lq[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 32; j += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int jj = j + u;
          acc[jj >> 3] = mfma32x32x16(op[jj % AHEAD], (jj & 15) < 8 ? kreg[jj & 7] : vreg[jj & 7], acc[jj >> 3]);
          if (jj + AHEAD < 32) op[jj % AHEAD] = operand(jj + AHEAD);
        }
        if (j == 8) {
          acc[3] = minus_d(1);
          log2_l(1, lq[1]);
        }
        if (j >= 16) pair(0, j - 16);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < 16; e += 2) pair(1, e);
    };
    auto produce_any = [&](int it, int qb, int pb) {
      if (is_full(it)) {
        if constexpr (DROP) produce(it, qb, pb, fast);
        else produce_full(it, qb, pb);
      } else {
        produce(it, qb, pb, general);
      }
    };
    if (it0 < it1) {
      if (it0 + 1 < it1) ld_load(it0 + 1);
      produce_any(it0, 0, 0);
      if (it0 + 1 < it1) ld_store(1);
      lds_barrier();
    }
    for (int it = it0; it < it1; ++it) {
      const int cur = (it - it0) & 1, nxt = cur ^ 1;
      const bool has_next2 = it + 2 < it1;
      if (has_next2) ld_load(it + 2);
      if (it + 1 < it1) produce_any(it + 1, nxt, nxt);
      if (has_next2) ld_store(cur);
      lds_barrier();
    }
  } else {
    const int n0 = 32 * role;  // this consumer's columns of dV and dK
    f32x16 acc_v[4], acc_k[4];  // one 32-key tile per key group
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc_v[m] = f32x16{};
      acc_k[m] = f32x16{};
    }
    if (it0 < it1) {
      dma_tile(it0, 0);
      if (it0 + 1 < it1) dma_tile(it0 + 1, 1);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    lds_barrier();
    // B operands (dO and Q read transposed for this consumer's column slice)
    // of the block being consumed, in registers: they are read from that
    // block's tile during the iteration before, so a tile is dead once the
    // producers have formed its block and the next tile can replace it
    // during the iteration, with one barrier per block.
    // Transposed reads of a swizzled tile: lane l gets rows 16 ks + 8 g +
    // (0..3) (and + 4..7) of column n0 + l % 32 (the lane's 8-byte read: row
    // r0 + j / 4, columns n0 + 16 ((l / 16) % 2) + 4 (j % 4) .. + 3, j = l % 16,
    // which stay in one 16-byte chunk; rows 16 ks + r share r's swizzle).
    int tro[2];
    {
      const int j = lane & 15;
      const int chunk = (n0 >> 3) + 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int r = 8 * g + 4 * x + (j >> 2);
        tro[x] = r * D + 8 * (chunk ^ tile_swz(r)) + 4 * (j & 1);
      }
    }
    e16x8 bo_r[C::BR / 16], bq_r[C::BR / 16];
    auto read_b = [&](int qb, int ks) {
      const int ro = 16 * ks * D;
      bo_r[ks] = concat(lds_read_tr(sO(qb) + ro + tro[0]), lds_read_tr(sO(qb) + ro + tro[1]));
      bq_r[ks] = concat(lds_read_tr(sQ(qb) + ro + tro[0]), lds_read_tr(sQ(qb) + ro + tro[1]));
    };
    // acc += A^T B over a block's queries, A = P~ (dV) or dS (dK) read
    // key-major from buffer pb; each k-step's B operands are then replaced by
    // those of the next block (tile qn; after the last block that tile holds
    // an older block, read but never used: no branch splits the loop)
    // The A operands of k-step ks + 1 are requested before the products of
    // k-step ks (two sets in flight), each step fenced.
    auto consume = [&](int pb, int qn) {
      const e16* Pt = sP(pb);
      const e16* St = sS(pb);
      e16x8 pa[2][4], sa[2][4];
      auto read_a = [&](int ks) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int off = (32 * m + c) * C::LDP + 16 * ks + 8 * g;
          pa[ks & 1][m] = load8(Pt + off);
          sa[ks & 1][m] = load8(St + off);
        }
      };
      read_a(0);
#pragma unroll
      for (int ks = 0; ks < C::BR / 16; ++ks) {  // 16-query k-steps
        if (ks + 1 < C::BR / 16) read_a(ks + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc_v[m] = mfma32x32x16(pa[ks & 1][m], bo_r[ks], acc_v[m]);
          acc_k[m] = mfma32x32x16(sa[ks & 1][m], bq_r[ks], acc_k[m]);
        }
        read_b(qn, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (it0 < it1) {
#pragma unroll
      for (int ks = 0; ks < C::BR / 16; ++ks) read_b(0, ks);
      lds_barrier();
    }
    for (int it = it0; it < it1; ++it) {
      const int cur = (it - it0) & 1, nxt = cur ^ 1;
      const bool has_next2 = it + 2 < it1;
      if (has_next2) dma_tile(it + 2, cur);
      consume(cur, nxt);
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
      lds_barrier();
    }
    // dK = sm_scale dS^T Q and dV = (Z o P)^T dO / (1 - p), rounded once to
    // the element type: each consumer writes its slices row-major into LDS
    // (free after the loop's last barrier); after the barrier below every
    // thread stores whole 8-column chunks with 16-byte stores.
    constexpr int SR = D + 8;
    static_assert(2 * C::BC * SR <= 4 * TILE + 4 * PT, "both outputs must fit the LDS staging");
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
        smem[row * SR + n0 + c] = (e16)(acc_v[m][r] * a.m.keep_scale);
        smem[(C::BC + row) * SR + n0 + c] = (e16)(acc_k[m][r] * (a.sm_scale * a.m.keep_scale));
      }
  }

  constexpr int SR = D + 8, CPR = D / 8;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2 * C::BC * CPR / C::NT; ++x) {
    const int chunk = tid + x * C::NT;
    const int row = chunk / CPR, col = (chunk % CPR) * 8;  // rows [0, BC): dV, [BC, 2 BC): dK
    const int kr = kv0 + (row & (C::BC - 1));
    if (kr < NK)
      store8(at<e16>(row < C::BC ? a.dv : a.dk, b, h, kr) + col, *(const e16x8*)(smem + row * SR + col));
  }
}

template <int D, bool DROP>
__global__ void __launch_bounds__(512) dkdv_ws_kernel(BwdArgs a) {
  int bh, blk;
  wg_coords(a.m.cu_q != nullptr, bh, blk);
  dkdv_ws_body<D, DROP>(a, bh, blk);
}

}  // namespace

hipError_t launch_kv128(const BwdArgs& a, hipStream_t s) {
  const int bh = a.B * a.H;
  const dim3 grid(bh, grid_blocks(bh, a.m.nk, KvSCfg<128>::BC, a.m.cu_q != nullptr));
  hipLaunchKernelGGL(a.m.dropout ? (dkdv_ws_kernel<128, true>) : (dkdv_ws_kernel<128, false>), grid,
                     dim3(KvSCfg<128>::NT), 0, s, a);
  return hipGetLastError();
}

FA_ELEM_NS_END
}  // namespace fa
