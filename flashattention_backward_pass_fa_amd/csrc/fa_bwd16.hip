// fa_bwd16.hip - 16-bit (bf16 or fp16) FlashAttention backward for gfx950
// (MFMA 32x32x16).  Compiled once per element type (see fa_device.h).
//
// The backward as a KV-outer and a Q-outer pass ("FlashAttention backward",
// section "The loop structure"):
//
//  dkdv_q2_kernel  KV-outer (deterministic mode, d = 64; d = 128 uses the
//                  producer/consumer kernel of fa_kv128.hip): one workgroup
//                  owns 128 keys of one (b, h) and loops over the 64-query blocks
//                  that can see them, with 8 waves (two per SIMD): 4 key
//                  groups x 2 query halves, K and V in LDS.  For each block
//                  it recomputes S = Q K^T and dP = dO V^T on MFMA, rebuilds
//                  P = exp(S - L) from the saved LSE ("Lecture 7", "The
//                  recomputation trick"), forms dS = P * (dP - D) with the
//                  pre-pass scalar D, and accumulates dV += P~^T dO and
//                  dK += dS^T Q in fp32 registers, written once at the end.
//  dkdv_atomic_kernel  KV-outer for atomic mode, 4 waves (32 keys each, K
//                  and V in registers): the same work, plus dS K added into
//                  an fp32 dQ accumulator with device atomics.
//  dq_kernel       Q-outer: 32 queries per wave (8 waves for d = 128, 4 for
//                  d = 64) streaming 32-key blocks through a ring of three
//                  LDS buffers, recomputing S, P, dP, dS to accumulate
//                  dQ = dS K in registers: the deterministic, atomic-free dQ.
//  bwd_small_kernel  both deterministic kernels' workgroups in one launch,
//                  for small fixed-length problems with d = 64 that would
//                  leave most of the chip idle one kernel at a time.
//
// Every kernel first specialises the call to its sequence (lengths, packed
// rows and the bottom-right alignment folded into the mask offsets).
//
// Layout in LDS: Q, dO, K, V tiles are row-major 16-bit with a padded row
// stride.  The k-inside-lane operands of the dV/dK/dQ products are read
// from those same tiles with ds_read_tr16_b64, so no transposed copies are
// kept.  Blocks that are fully masked (causal/window) are never visited; a
// wave whose 32x32 tile is fully masked skips its products; only tiles that
// straddle a mask edge or the sequence end evaluate the per-element mask,
// and the fully visible ones run a path ordered so that the exponentials
// and dS sit beside independent MFMAs.

#include <type_traits>

#include "fa_bwd_common.h"

namespace fa {
FA_ELEM_NS_BEGIN
namespace {

template <int D>
struct KvCfg {
  static constexpr int BC = 128;          // keys per workgroup
  static constexpr int BR = 64;           // queries per inner iteration
  static constexpr int NT = 256;          // threads (4 waves)
  static constexpr int LD = lds_stride(D);  // LDS row stride of Q/dO/K tiles
  static constexpr int LDS_T = BR + 8;     // LDS row stride of the dS^T tile (36 dwords)
  static constexpr int KT = D / 16;       // MFMA k-steps over d
  static constexpr int DT = D / 32;       // 32-wide tiles over d
  static constexpr int CH = D / 8;        // 16-byte chunks per row
  static constexpr int LOADS = BR * CH / NT;
};


// Elementwise step of one 32x32 S/dP accumulator pair of the KV-outer kernel:
// P = exp2(S * c - L2), masked, dropout, dS = P (dP - D).  Writes the 16-bit
// A operands of dV (P~) and dK (dS) for the two 16-query k-steps.  With
// dropout (DROPNOW) it writes dS (1 - p) = P~ dP - P D (1 - p) instead:
// 1 / (1 - p) is applied to dV and dK at the store, and sDq holds D (1 - p).
template <bool GENERAL, bool DROPNOW>
__device__ __forceinline__ void kv_elementwise_body(const BwdArgs& a, const f32x16& s, const f32x16& dp,
                                                    const float* sLq, const float* sDq, int g, int b,
                                                    int h, int q0, int key, e16x8& pa0, e16x8& pa1,
                                                    e16x8& da0, e16x8& da1) {
  // Dropout: keys across lanes, so the eight lanes of a Philox block share
  // each row's block (bit 8 rr + t of kq[e]: row 8 rr + 4 g + e; t: the
  // key's bit in a byte of the traded words)
  uint32_t kq[4] = {~0u, ~0u, ~0u, ~0u};
  const int t = dropout_octet_bit(key);
  if (DROPNOW) dropout_keep_octet(a.m, b, h, q0, g, key, kq);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const f32x4 l4 = *(const f32x4*)(sLq + 8 * rr + 4 * g);
    const f32x4 d4 = *(const f32x4*)(sDq + 8 * rr + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * rr + e;
      float p = fast_exp2(s[r] * a.scale_log2 - l4[e]);
      if (GENERAL) p = visible(a.m, q0 + 8 * rr + 4 * g + e, key) ? p : 0.f;
      const float pdrop = DROPNOW ? masked(p, bit_mask(kq[e], 8 * rr + t)) : p;
      const float ds = DROPNOW ? fmaf(pdrop, dp[r], -(p * d4[e])) : p * (dp[r] - d4[e]);
      if (r < 8) {
        pa0[r] = (e16)pdrop;
        da0[r] = (e16)ds;
      } else {
        pa1[r - 8] = (e16)pdrop;
        da1[r - 8] = (e16)ds;
      }
    }
  }
}

template <bool GENERAL, bool DROPOK = true>
__device__ __forceinline__ void kv_elementwise(const BwdArgs& a, const f32x16& s, const f32x16& dp,
                                               const float* sLq, const float* sDq, int g, int b,
                                               int h, int q0, int key, e16x8& pa0, e16x8& pa1,
                                               e16x8& da0, e16x8& da1) {
  if (GENERAL && DROPOK && a.m.dropout)
    kv_elementwise_body<GENERAL, true>(a, s, dp, sLq, sDq, g, b, h, q0, key, pa0, pa1, da0, da1);
  else
    kv_elementwise_body<GENERAL, false>(a, s, dp, sLq, sDq, g, b, h, q0, key, pa0, pa1, da0, da1);
}

// One fully visible 32-query x 32-key tile of a KV-outer wave, without
// dropout, ordered so that VALU work has independent MFMAs beside it: S,
// then dP while P = exp2(S c - L) is formed, then dV += P^T dO while
// dS = P (dP - D) is formed, then dK += dS^T Q.  qrow/orow point at this
// lane's query row of the Q and dO tiles (at column 8 g), kr/vr at its key
// row of K and V; u0 is the first 16-query k-step of the tile.
template <int D, int LD, bool DROP, typename Mid>
__device__ __forceinline__ void kv_full_tile(const BwdArgs& a, const e16* qrow, const e16* orow,
                                             const e16* kr, const e16* vr, const e16* Qs,
                                             const e16* Os, const float* sLq, const float* sDq,
                                             int g, int lane, int u0, f32x16* dk_acc,
                                             f32x16* dv_acc, Mid mid, int b, int h, int qs,
                                             int key) {
  constexpr int KT = D / 16, DT = D / 32;
  const int ulo = 16 * u0 + 4 * g;  // first query row of this lane's k-steps
  f32x16 sacc = f32x16{};
#pragma unroll
  for (int t = 0; t < KT; ++t) sacc = mfma32x32x16(load8(qrow + 16 * t), load8(kr + 16 * t), sacc);
  mid();
  // dropout keep bits: the eight lanes of a Philox block share each row's
  // block (bit 8 rr + kt8 of kq[e]: row qs + 8 rr + 4 g + e; kt8: the key's
  // bit in a byte of the traded words)
  uint32_t kq[4] = {0u, 0u, 0u, 0u};
  const int kt8 = dropout_octet_bit(key);
  if (DROP) dropout_keep_octet(a.m, b, h, qs, g, key, kq);
  f32x16 dpacc = f32x16{};
#pragma unroll
  for (int t = 0; t < KT; ++t) dpacc = mfma32x32x16(load8(orow + 16 * t), load8(vr + 16 * t), dpacc);
  e16x8 b0[DT], b1[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) b0[n] = tr_operand(Os, LD, ulo, ulo + 8, 32 * n, lane);
  float p[16], pk[16];  // P and (dropout) P~ = P Z
  e16x8 pa[2], da[2];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const f32x4 l4 = *(const f32x4*)(sLq + 8 * rr + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * rr + e;
      p[r] = fast_exp2(sacc[r] * a.scale_log2 - l4[e]);
      pk[r] = DROP ? masked(p[r], bit_mask(kq[e], 8 * rr + kt8)) : p[r];
      pa[r >> 3][r & 7] = (e16)pk[r];  // 1 / (1 - p) at the dV store
    }
  }
#pragma unroll
  for (int n = 0; n < DT; ++n) b1[n] = tr_operand(Os, LD, ulo + 16, ulo + 24, 32 * n, lane);
#pragma unroll
  for (int n = 0; n < DT; ++n) dv_acc[n] = mfma32x32x16(pa[0], b0[n], dv_acc[n]);
#pragma unroll
  for (int n = 0; n < DT; ++n) dv_acc[n] = mfma32x32x16(pa[1], b1[n], dv_acc[n]);
#pragma unroll
  for (int n = 0; n < DT; ++n) b0[n] = tr_operand(Qs, LD, ulo, ulo + 8, 32 * n, lane);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const f32x4 d4 = *(const f32x4*)(sDq + 8 * rr + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * rr + e;
      // dropout: dS (1 - p) = P~ dP - P D (1 - p), with 1 / (1 - p) at the dK
      // store and D (1 - p) in sDq
      da[r >> 3][r & 7] = (e16)(DROP ? fmaf(pk[r], dpacc[r], -(p[r] * d4[e])) : p[r] * (dpacc[r] - d4[e]));
    }
  }
#pragma unroll
  for (int n = 0; n < DT; ++n) b1[n] = tr_operand(Qs, LD, ulo + 16, ulo + 24, 32 * n, lane);
#pragma unroll
  for (int n = 0; n < DT; ++n) dk_acc[n] = mfma32x32x16(da[0], b0[n], dk_acc[n]);
#pragma unroll
  for (int n = 0; n < DT; ++n) dk_acc[n] = mfma32x32x16(da[1], b1[n], dk_acc[n]);
}

// ---------------------------------------------------- KV-outer, atomic dQ

template <int D>
__global__ void __launch_bounds__(256, 1) dkdv_atomic_kernel(BwdArgs a) {
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(16))) e16 sQ[2][C::BR * C::LD];
  __shared__ __attribute__((aligned(16))) e16 sO[2][C::BR * C::LD];
  __shared__ __attribute__((aligned(16))) e16 sK[C::BC * C::LD];
  __shared__ __attribute__((aligned(16))) e16 sT[C::BC * C::LDS_T];
  __shared__ __attribute__((aligned(16))) float sL[2][C::BR];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  int bh, blk;
  wg_coords(a.m.cu_q != nullptr, bh, blk);
  const int b = bh / a.H, h = bh - b * a.H;
  bwd_localize(a, b);
  const int NQ = a.m.nq, NK = a.m.nk;
  const int kv0 = blk * C::BC;
  if (kv0 >= NK) return;  // past this sequence's keys
  const int kvw = kv0 + 32 * w;
  const int key = kvw + c;  // this lane's key (column of S)

  // Query rows that can see at least one of the block's keys.
  const int q_lo = max(0, kv0 - a.m.hi_off), q_hi = min(NQ, kv0 + C::BC + a.m.lo_off);
  const int it0 = q_lo / C::BR;
  const int it1 = q_lo < q_hi ? (q_hi + C::BR - 1) / C::BR : it0;

  const int64_t row_base = (int64_t)bh * a.ln;
  e16x8 pq[C::LOADS], po[C::LOADS];
  float pl = 0.f, pd = 0.f;

  auto load_tile = [&](int it) {
    const int q0 = it * C::BR;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int qc = min(q0 + row, NQ - 1);
      pq[x] = load8(at<e16>(a.q, b, h, qc) + col);
      po[x] = load8(at<e16>(a.dout, b, h, qc) + col);
    }
    const int qc = min(q0 + (tid & (C::BR - 1)), NQ - 1);  // every thread loads; tid < BR stores
    pl = a.lse[row_base + qc];  // scaled at the store: arithmetic here would wait for the load
    pd = a.delta[row_base + qc];
  };
  if (it0 < it1) load_tile(it0);  // in flight with the K, V loads below

  // This wave's 32 keys: B operands of S = Q K^T and dP = dO V^T.
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
  // the block's K rows, row-major in LDS: B operand of dQ = dS K
  {
    constexpr int KL = C::BC * C::CH / C::NT;
    e16x8 kx[KL];
#pragma unroll
    for (int x = 0; x < KL; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      kx[x] = load8(at<e16>(a.k, b, h, min(kv0 + row, NK - 1)) + col);
    }
#pragma unroll
    for (int x = 0; x < KL; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(sK + row * C::LD + col, kx[x]);
    }
  }
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(&sQ[buf][row * C::LD + col], pq[x]);
      store8(&sO[buf][row * C::LD + col], po[x]);
    }
    if (tid < C::BR) {
      sL[buf][tid] = pl * kLog2e;
      sD[buf][tid] = pd / a.m.keep_scale;  // D (1 - p): exactly D without dropout
    }
  };

  f32x16 dk_acc[C::DT], dv_acc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) {
    dk_acc[n] = f32x16{};
    dv_acc[n] = f32x16{};
  }

  if (it0 < it1) store_tile(0);
  __syncthreads();

  for (int it = it0; it < it1; ++it) {
    const int buf = (it - it0) & 1;
    const bool has_next = it + 1 < it1;
    if (has_next) load_tile(it + 1);
    const e16* Qs = sQ[buf];
    const e16* Os = sO[buf];
    const int q0 = it * C::BR;

#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int qs = q0 + 32 * qt;  // first query of this 32-query sub-tile
      e16x8 pa0, pa1, da0, da1;
      if (!block_dead(a.m, qs, 32, kvw, 32)) {
        // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
        e16x8 aq[C::KT], ao[C::KT];
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
          aq[t] = load8(Qs + (32 * qt + c) * C::LD + 16 * t + 8 * g);
          ao[t] = load8(Os + (32 * qt + c) * C::LD + 16 * t + 8 * g);
        }
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
          s = mfma32x32x16(aq[t], kreg[t], s);
          dp = mfma32x32x16(ao[t], vreg[t], dp);
        }
        const float* sLq = &sL[buf][32 * qt];
        const float* sDq = &sD[buf][32 * qt];
        if (block_full(a.m, qs, 32, kvw, 32) && !a.m.dropout)
          kv_elementwise<false>(a, s, dp, sLq, sDq, g, b, h, qs, key, pa0, pa1, da0, da1);
        else
          kv_elementwise<true>(a, s, dp, sLq, sDq, g, b, h, qs, key, pa0, pa1, da0, da1);

        // dV += P~^T dO and dK += dS^T Q over these 32 queries
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          const int u = 2 * qt + u2;
          e16x8 bo[C::DT], bq[C::DT];
#pragma unroll
          for (int n = 0; n < C::DT; ++n) {
            bo[n] = tr_operand(Os, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
            bq[n] = tr_operand(Qs, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
          }
#pragma unroll
          for (int n = 0; n < C::DT; ++n) {
            dv_acc[n] = mfma32x32x16(u2 ? pa1 : pa0, bo[n], dv_acc[n]);
            dk_acc[n] = mfma32x32x16(u2 ? da1 : da0, bq[n], dk_acc[n]);
          }
        }
      } else {
        da0 = zero8();
        da1 = zero8();
      }
      // dS^T of this wave's keys into LDS: sT[key][query]
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const e16x8 src = rr < 2 ? da0 : da1;
        const int s0 = (rr & 1) * 4;
        const e16x4 v4 = {src[s0], src[s0 + 1], src[s0 + 2], src[s0 + 3]};
        *(e16x4*)(sT + (32 * w + c) * C::LDS_T + 32 * qt + 8 * rr + 4 * g) = v4;
      }
    }

    {
      lds_barrier();
      // dQ partial of the 64 queries over the block's 128 keys
      constexpr int MT = D == 128 ? 2 : 1;  // 32-query tiles per wave
      const int nt = D == 128 ? w : (w & 1);
      const int mt0 = D == 128 ? 0 : (w >> 1);
      f32x16 dq[MT];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) dq[mi] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::BC / 16; ++t) {
        const e16x8 bk = tr_operand(sK, C::LD, 16 * t + 8 * g, 16 * t + 8 * g + 4, 32 * nt, lane);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          const e16x8 as =
              tr_operand(sT, C::LDS_T, 16 * t + 8 * g, 16 * t + 8 * g + 4, 32 * (mt0 + mi), lane);
          dq[mi] = mfma32x32x16(as, bk, dq[mi]);
        }
      }
      // The next tile's loads are consumed before this step's atomics are
      // issued, so waiting for them never waits for the atomics' round trip.
      if (has_next) store_tile(buf ^ 1);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = q0 + 32 * (mt0 + mi) + 8 * (r >> 2) + 4 * g + (r & 3);
          if (qr < NQ) unsafeAtomicAdd(a.dq_acc + (row_base + qr) * D + 32 * nt + c, dq[mi][r]);
        }
      }
    }
    lds_barrier();
  }

  // dK = sm_scale * dS^T Q, dV = (Z o P)^T dO / (1 - p): one rounding to the element type at the store.
#pragma unroll
  for (int n = 0; n < C::DT; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kvw + 8 * (r >> 2) + 4 * g + (r & 3);
      if (kr < NK) {
        at<e16>(a.dk, b, h, kr)[32 * n + c] = (e16)(dk_acc[n][r] * (a.sm_scale * a.m.keep_scale));
        at<e16>(a.dv, b, h, kr)[32 * n + c] = (e16)(dv_acc[n][r] * a.m.keep_scale);
      }
    }
  }
}

// ------------------------------------------- KV-outer, queries split by wave

// KV-outer kernel with 8 independent waves (two per SIMD).  The workgroup's
// 128 keys are 4 groups of 32; wave w takes key group w % 4 and query half
// w / 4 of every 64-query block, and accumulates its own partial dK, dV.
// K and V of the block sit in LDS (B operands of S and dP read with b128),
// so a wave holds only its 32 x d dK and dV accumulators: it fits in 256
// registers.  The two partials of a key group are summed through LDS once,
// after the loop.
template <int D>
struct KvQCfg {
  static constexpr int BC = 128, BR = 64, NT = 512;
  static constexpr int LD = lds_stride(D);
  static constexpr int KT = D / 16, DT = D / 32, CH = D / 8;
  static constexpr int LOADS = BR * CH / NT;        // Q (and dO) chunks per thread per block
  static constexpr int KV_LOADS = BC * CH / NT;     // K (and V) chunks per thread, once
};

template <int D, bool DROP>
__device__ __forceinline__ void dkdv_q2_body(BwdArgs& a, int bh, int blk) {
  using C = KvQCfg<D>;
  // [0, 4*BR*LD): Q, dO double buffers; then K and V; reused for the
  // partial-sum exchange after the loop.
  constexpr int TILE = C::BR * C::LD, KVT = C::BC * C::LD;
  __shared__ __attribute__((aligned(16))) e16 smem[4 * TILE + 2 * KVT];
  __shared__ __attribute__((aligned(16))) float sL[2][C::BR];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BR];
  // Q buffers at smem + buf * TILE, dO buffers at smem + (2 + buf) * TILE
  e16* sK = smem + 4 * TILE;
  e16* sV = sK + KVT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int grp = w & 3, qh = w >> 2;
  const int b = bh / a.H, h = bh - b * a.H;
  bwd_localize(a, b);
  const int NQ = a.m.nq, NK = a.m.nk;
  const int kv0 = blk * C::BC;
  if (kv0 >= NK) return;  // past this sequence's keys
  const int kvw = kv0 + 32 * grp;
  const int key = kvw + c;

  // Query rows that can see at least one of the block's keys.
  const int q_lo = max(0, kv0 - a.m.hi_off), q_hi = min(NQ, kv0 + C::BC + a.m.lo_off);
  const int it0 = q_lo / C::BR;
  const int it1 = q_lo < q_hi ? (q_hi + C::BR - 1) / C::BR : it0;

  const int64_t row_base = (int64_t)bh * a.ln;
  const char* q_head = (const char*)at<e16>(a.q, b, h, 0);
  const char* o_head = (const char*)at<e16>(a.dout, b, h, 0);
  const uint32_t q_rs = (uint32_t)a.q.sn * 2, o_rs = (uint32_t)a.dout.sn * 2;
  e16x8 pq[C::LOADS], po[C::LOADS];
  float pld = 0.f;
  auto load_tile = [&](int it) {
    const int q0 = it * C::BR;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int qr = min(q0 + row, NQ - 1);  // rows past the end are masked: read a valid one
      pq[x] = load8((const e16*)row_addr(q_head, q_rs, qr) + col);
      po[x] = load8((const e16*)row_addr(o_head, o_rs, qr) + col);
    }
    if (tid < 2 * C::BR)
      pld = (tid < C::BR ? a.lse : a.delta)[row_base + min(q0 + (tid & (C::BR - 1)), NQ - 1)];
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(smem + buf * TILE + row * C::LD + col, pq[x]);
      store8(smem + (2 + buf) * TILE + row * C::LD + col, po[x]);
    }
    if (tid < C::BR) sL[buf][tid] = pld * kLog2e;
    else if (tid < 2 * C::BR) sD[buf][tid - C::BR] = pld / a.m.keep_scale;  // D (1 - p): exactly D without dropout
  };

  f32x16 dk_acc[C::DT], dv_acc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) {
    dk_acc[n] = f32x16{};
    dv_acc[n] = f32x16{};
  }

  // The first Q/dO block and the block's K and V rows are all loaded before
  // anything is stored, so the prologue waits for memory once.
  if (it0 < it1) load_tile(it0);
  {
    e16x8 kx[C::KV_LOADS], vx[C::KV_LOADS];
#pragma unroll
    for (int x = 0; x < C::KV_LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int kc = min(kv0 + row, NK - 1);
      kx[x] = load8(at<e16>(a.k, b, h, kc) + col);
      vx[x] = load8(at<e16>(a.v, b, h, kc) + col);
    }
#pragma unroll
    for (int x = 0; x < C::KV_LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(sK + row * C::LD + col, kx[x]);
      store8(sV + row * C::LD + col, vx[x]);
    }
  }
  if (it0 < it1) store_tile(0);
  __syncthreads();

  const e16* Kr = sK + (32 * grp + c) * C::LD + 8 * g;  // this lane's key row (B operands)
  const e16* Vr = sV + (32 * grp + c) * C::LD + 8 * g;
  // FULL: every wave's tile fully visible; PRE: the next block exists and is
  // loaded from inside the tile's products
  auto step = [&](int it, auto full, auto pre, auto drop) {
    const int buf = (it - it0) & 1;
    const bool has_next = it + 1 < it1;
    if (!decltype(pre)::value && has_next) load_tile(it + 1);
    const e16* Qs = smem + buf * TILE;
    const e16* Os = smem + (2 + buf) * TILE;
    const int qs = it * C::BR + 32 * qh;
    if (decltype(full)::value) {
      kv_full_tile<D, C::LD, decltype(drop)::value>(
          a, Qs + (32 * qh + c) * C::LD + 8 * g, Os + (32 * qh + c) * C::LD + 8 * g, Kr, Vr, Qs, Os,
          &sL[buf][32 * qh], &sD[buf][32 * qh], g, lane, 2 * qh, dk_acc, dv_acc,
          [&] { if (decltype(pre)::value) load_tile(it + 1); }, b, h, qs, key);
    } else if (!block_dead(a.m, qs, 32, kvw, 32)) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int t = 0; t < C::KT; ++t) {
        const e16x8 aq = load8(Qs + (32 * qh + c) * C::LD + 16 * t + 8 * g);
        const e16x8 ao = load8(Os + (32 * qh + c) * C::LD + 16 * t + 8 * g);
        sacc = mfma32x32x16(aq, load8(Kr + 16 * t), sacc);
        dpacc = mfma32x32x16(ao, load8(Vr + 16 * t), dpacc);
      }
      e16x8 pa0, pa1, da0, da1;
      const float* sLq = &sL[buf][32 * qh];
      const float* sDq = &sD[buf][32 * qh];
      kv_elementwise_body<true, DROP>(a, sacc, dpacc, sLq, sDq, g, b, h, qs, key, pa0, pa1, da0, da1);  // launched with dropout on iff DROP
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = 2 * qh + u2;
        e16x8 bo[C::DT], bq[C::DT];
#pragma unroll
        for (int n = 0; n < C::DT; ++n) {
          bo[n] = tr_operand(Os, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
          bq[n] = tr_operand(Qs, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
        }
#pragma unroll
        for (int n = 0; n < C::DT; ++n) {
          dv_acc[n] = mfma32x32x16(u2 ? pa1 : pa0, bo[n], dv_acc[n]);
          dk_acc[n] = mfma32x32x16(u2 ? da1 : da0, bq[n], dk_acc[n]);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    lds_barrier();
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
  std::integral_constant<bool, false> general;
  std::integral_constant<bool, true> fast;
  std::integral_constant<bool, false> no_pre, no_drop;
  std::integral_constant<bool, true> pre, drop;
  int it = it0;
  for (; it < itA; ++it) step(it, general, no_pre, no_drop);
  if (DROP) {
    for (; it < min(itB, it1 - 1); ++it) step(it, fast, pre, drop);
    for (; it < itB; ++it) step(it, fast, no_pre, drop);
  } else {
    for (; it < min(itB, it1 - 1); ++it) step(it, fast, pre, no_drop);
    for (; it < itB; ++it) step(it, fast, no_pre, no_drop);
  }
  for (; it < it1; ++it) step(it, general, no_pre, no_drop);

  // dK and dV, one after the other: both query halves write their fp32
  // partials row-major into LDS (the tiles are free after the loop's last
  // barrier), then every thread adds the two halves of whole 8-column chunks
  // and writes them with one 16-byte store (stores of single elements from
  // the accumulator layout cost most of the kernel's fixed time).  Row
  // stride XS = D + 8 floats puts the two row groups a wave writes at once
  // (rows r and r + 4) on opposite halves of the banks.
  constexpr int XS = D + 8, CPR = D / 8;  // floats per row, 8-column chunks per row
  static_assert(2 * C::BC * XS * 4 <= (4 * TILE + 2 * KVT) * 2, "partials must fit the tiles' LDS");
  float* part = (float*)smem;  // [2 halves][BC keys][XS]
  auto finish = [&](const f32x16* acc, const TensorView& out, float scale) {
#pragma unroll
    for (int n = 0; n < C::DT; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        part[(qh * C::BC + 32 * grp + 8 * (r >> 2) + 4 * g + (r & 3)) * XS + 32 * n + c] = acc[n][r];
    __syncthreads();
#pragma unroll
    for (int x = 0; x < C::BC * CPR / C::NT; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / CPR, col = (chunk % CPR) * 8;
      const float* p0 = part + row * XS + col;
      const float* p1 = part + (C::BC + row) * XS + col;
      const f32x4 a0 = *(const f32x4*)p0, a1 = *(const f32x4*)(p0 + 4);
      const f32x4 b0 = *(const f32x4*)p1, b1 = *(const f32x4*)(p1 + 4);
      e16x8 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = (e16)((a0[e] + b0[e]) * scale);
        v[4 + e] = (e16)((a1[e] + b1[e]) * scale);
      }
      if (kv0 + row < NK) store8(at<e16>(out, b, h, kv0 + row) + col, v);
    }
    __syncthreads();
  };
  finish(dk_acc, a.dk, a.sm_scale * a.m.keep_scale);  // dropout: dS (1 - p) was accumulated
  finish(dv_acc, a.dv, a.m.keep_scale);  // 1 / (1 - p): exactly 1 without dropout
}

template <int D, bool DROP>
__global__ void __launch_bounds__(512) dkdv_q2_kernel(BwdArgs a) {
  int bh, blk;
  wg_coords(a.m.cu_q != nullptr, bh, blk);
  dkdv_q2_body<D, DROP>(a, bh, blk);
}

// ---------------------------------------------------------------- Q-outer

// Q-outer dQ kernel with 32-key blocks streamed through a ring of three LDS
// buffers, so that one block's S^T, dP^T products can run while the previous
// block's dS is formed.  Block j + 2 is loaded into registers while block j
// is worked on and lands in the buffer block j - 1 used.  Over key blocks
// that the whole workgroup sees without a mask edge (and without dropout)
// each iteration issues S^T, dP^T of block j + 1 beside the exponentials and
// dS of block j, then dQ += dS K of block j; other blocks run the plain
// per-block sequence with the mask.
template <int D, int NT_ = (D == 128 ? 512 : 256)>
struct QCfg {
  static constexpr int NT = NT_, BQ = NT / 2, BK = 32;
  static constexpr int MINB = 512 / NT;
  static constexpr int LD = lds_stride(D);
  static constexpr int KT = D / 16, DT = D / 32, CH = D / 8;
  // 16-byte chunks of one 32-key tile; with more threads than chunks the
  // threads past them move nothing
  static constexpr int TILE_CHUNKS = BK * CH;
  static constexpr int LOADS = (TILE_CHUNKS + NT - 1) / NT;
};

template <int D, bool DROP, int NT>
__device__ __forceinline__ void dq_body(BwdArgs& a, int bh, int blk) {
  using C = QCfg<D, NT>;
  // the K and V rings (three blocks each), one array so that the final dQ
  // rows can be staged through it
  __shared__ __attribute__((aligned(16))) e16 kv_ring[6][C::BK * C::LD];
  e16 (*sK)[C::BK * C::LD] = kv_ring;
  e16 (*sV)[C::BK * C::LD] = kv_ring + 3;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int b = bh / a.H, h = bh - b * a.H;
  bwd_localize(a, b);
  const int NQ = a.m.nq, NK = a.m.nk;
  // Longest first: with a causal mask the last query blocks see the most keys.
  const int nblk = (NQ + C::BQ - 1) / C::BQ;
  if (blk >= nblk) return;  // past this sequence's queries
  const int qblk = a.m.causal ? nblk - 1 - blk : blk;
  const int q0 = qblk * C::BQ;
  const int qw = q0 + 32 * w;
  const int myq = qw + c;
  const int64_t row_base = (int64_t)bh * a.ln;

  // This wave's 32 queries: B operands of S^T = K Q^T and dP^T = V dO^T.
  e16x8 qreg[C::KT], oreg[C::KT];
  {
    const bool ok = myq < NQ;
    const e16* qp = at<e16>(a.q, b, h, ok ? myq : 0);
    const e16* op = at<e16>(a.dout, b, h, ok ? myq : 0);
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
      qreg[t] = ok ? load8(qp + 16 * t + 8 * g) : zero8();
      oreg[t] = ok ? load8(op + 16 * t + 8 * g) : zero8();
    }
  }
  const float l2 = myq < NQ ? a.lse[row_base + myq] * kLog2e : 0.f;
  const float dd = myq < NQ ? a.delta[row_base + myq] : 0.f;

  // Keys that at least one of the block's queries can see.
  const int k_lo = max(0, q0 - a.m.lo_off), k_hi = min(NK, q0 + C::BQ + a.m.hi_off);
  const int jt0 = k_lo / C::BK;
  const int jt1 = k_lo < k_hi ? (k_hi + C::BK - 1) / C::BK : jt0;

  const char* k_head = (const char*)at<e16>(a.k, b, h, 0);
  const char* v_head = (const char*)at<e16>(a.v, b, h, 0);
  const uint32_t k_rs = (uint32_t)a.k.sn * 2, v_rs = (uint32_t)a.v.sn * 2;
  e16x8 pk[C::LOADS], pv[C::LOADS];
  auto load_into = [&](int jt, e16x8* kd, e16x8* vd) {
    const int k0 = jt * C::BK;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      if (C::TILE_CHUNKS % C::NT != 0 && chunk >= C::TILE_CHUNKS) break;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int kr = min(k0 + row, NK - 1);
      kd[x] = load8((const e16*)row_addr(k_head, k_rs, kr) + col);
      vd[x] = load8((const e16*)row_addr(v_head, v_rs, kr) + col);
    }
  };
  auto store_from = [&](int buf, const e16x8* ks, const e16x8* vs) {
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      if (C::TILE_CHUNKS % C::NT != 0 && chunk >= C::TILE_CHUNKS) break;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(&sK[buf][row * C::LD + col], ks[x]);
      store8(&sV[buf][row * C::LD + col], vs[x]);
    }
  };
  auto load_tile = [&](int jt) { load_into(jt, pk, pv); };
  auto store_tile = [&](int buf) { store_from(buf, pk, pv); };
  auto ring = [&](int jt) { return (jt - jt0) % 3; };

  f32x16 dq_acc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) dq_acc[n] = f32x16{};

  // dP^T accumulates from -D, so that without dropout the product ends as
  // dP - D; with dropout from -D (1 - p), so that it ends as
  // (dP / (1 - p) - D) (1 - p) for a kept element, and a dropped one's
  // -D (1 - p) is the start value itself: the wave forms dS (1 - p), and the
  // dQ store applies 1 / (1 - p)
  f32x16 dp0;
  {
    const float start = DROP ? -dd / a.m.keep_scale : -dd;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp0[r] = start;
  }
  // S^T, dP^T of one 32-key block against this wave's queries
  auto sdp = [&](int buf, f32x16& st, f32x16& dpt) {
    st = f32x16{};
    dpt = dp0;
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
      st = mfma32x32x16(load8(&sK[buf][c * C::LD + 16 * t + 8 * g]), qreg[t], st);
      dpt = mfma32x32x16(load8(&sV[buf][c * C::LD + 16 * t + 8 * g]), oreg[t], dpt);
    }
  };
  auto dqmm = [&](int buf, const e16x8& d0, const e16x8& d1) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int n = 0; n < C::DT; ++n)
        dq_acc[n] = mfma32x32x16(u ? d1 : d0, tr_operand(sK[buf], C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane),
                                 dq_acc[n]);
    }
  };
  // The start of every iteration publishes block jt + 2, whose loads were
  // issued one iteration earlier (its buffer held block jt - 1, free since
  // the last barrier; it is first read after this iteration's barrier), and
  // issues block jt + 3's loads.
  auto prefetch = [&](int jt) {
    if (jt + 2 < jt1) store_tile(ring(jt + 2));
    if (jt + 3 < jt1) load_tile(jt + 3);
  };

  if (jt0 < jt1) {
    e16x8 k0[C::LOADS], v0[C::LOADS], k1[C::LOADS], v1[C::LOADS];
    load_into(jt0, k0, v0);
    if (jt0 + 1 < jt1) load_into(jt0 + 1, k1, v1);
    if (jt0 + 2 < jt1) load_tile(jt0 + 2);
    store_from(0, k0, v0);
    if (jt0 + 1 < jt1) store_from(1, k1, v1);
  }
  __syncthreads();

  // Key blocks [jtA, jtB) are seen by all of the block's queries with no
  // mask edge.  Query rows past the sequence end need no mask: their Q and
  // dO are zero, so they only add dS = 0 to their own (unstored) dQ rows;
  // the last real row bounds the left window.
  int jtA = jt1, jtB = jt1;
  {
    const int qlast = min(q0 + C::BQ, NQ) - 1;
    const int lo = max(0, qlast - a.m.lo_off);
    const int hi = min(NK - C::BK, q0 + a.m.hi_off - C::BK + 1);
    if (lo <= hi) {
      jtA = min(max(jt0, (lo + C::BK - 1) / C::BK), jt1);
      jtB = max(jtA, min(jt1, hi / C::BK + 1));
    }
  }

  auto general = [&](int jt) {
    prefetch(jt);
    const int buf = ring(jt);
    const int ks = jt * C::BK;
    if (!block_dead(a.m, qw, 32, ks, 32)) {
      f32x16 st, dpt;
      sdp(buf, st, dpt);
      e16x8 d0, d1;
      // this lane's keys ks + 8 rr + 4 g + (0..3) at bits 4 rr + (0..3)
      const uint32_t kp = DROP ? dropout_keep_lane(a.m, b, h, myq, ks, g) : ~0u;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int j4 = ks + 8 * rr + 4 * g;
        const uint32_t keep = (kp >> (4 * rr)) & 0xFu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          float p = fast_exp2(st[r] * a.scale_log2 - l2);
          float dmd = dpt[r];  // dP - D (dropout: with dP scaled by 1 - p)
          p = visible(a.m, myq, j4 + e) ? p : 0.f;
          if (DROP) dmd = (keep >> e) & 1u ? dmd : dp0[0];  // dS (1 - p): 1 / (1 - p) at the dQ store
          const e16 v = (e16)(p * dmd);
          if (r < 8) d0[r] = v; else d1[r - 8] = v;
        }
      }
      dqmm(buf, d0, d1);
    }
    lds_barrier();
  };

  int jt = jt0;
  for (; jt < jtA; ++jt) general(jt);
  // the fully visible range, software-pipelined; DROP: with the dropout mask
  auto fast_range = [&](auto drop) {
    constexpr bool FDROP = decltype(drop)::value;
    auto ds_of = [&](int j, const f32x16& st, const f32x16& dpt, e16x8& d0, e16x8& d1) {
      const uint32_t kp = FDROP ? dropout_keep_lane(a.m, b, h, myq, j * C::BK, g) : ~0u;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t keep = (kp >> (4 * rr)) & 0xFu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          float dmd = dpt[r];
          if (FDROP) dmd = (keep >> e) & 1u ? dmd : dp0[0];  // dS (1 - p): 1 / (1 - p) at the dQ store
          const e16 v = (e16)(fast_exp2(st[r] * a.scale_log2 - l2) * dmd);
          if (r < 8) d0[r] = v; else d1[r - 8] = v;
        }
      }
    };
    f32x16 st, dpt;
    sdp(ring(jtA), st, dpt);
    for (; jt + 1 < jtB; ++jt) {
      prefetch(jt);
      f32x16 st_n, dpt_n;
      sdp(ring(jt + 1), st_n, dpt_n);
      const e16* Kc = sK[ring(jt)];
      e16x8 b0[C::DT], b1[C::DT];
#pragma unroll
      for (int n = 0; n < C::DT; ++n) b0[n] = tr_operand(Kc, C::LD, 4 * g, 8 + 4 * g, 32 * n, lane);
      e16x8 d0, d1;
      ds_of(jt, st, dpt, d0, d1);
#pragma unroll
      for (int n = 0; n < C::DT; ++n) b1[n] = tr_operand(Kc, C::LD, 16 + 4 * g, 24 + 4 * g, 32 * n, lane);
#pragma unroll
      for (int n = 0; n < C::DT; ++n) dq_acc[n] = mfma32x32x16(d0, b0[n], dq_acc[n]);
#pragma unroll
      for (int n = 0; n < C::DT; ++n) dq_acc[n] = mfma32x32x16(d1, b1[n], dq_acc[n]);
      lds_barrier();
      st = st_n;
      dpt = dpt_n;
    }
    prefetch(jt);
    e16x8 d0, d1;
    ds_of(jt, st, dpt, d0, d1);
    dqmm(ring(jt), d0, d1);
    lds_barrier();
    ++jt;
  };
  // With dropout at d = 128 the pipelined range's second set of S^T, dP^T
  // accumulators and the Philox state do not fit beside the rest without
  // spilling: every block then takes the per-block sequence.
  if (jtA < jtB && !(DROP && D == 128)) fast_range(std::integral_constant<bool, DROP>());
  for (; jt < jt1; ++jt) general(jt);

  // dQ = sm_scale dS K: the waves write their rows (rounded) row-major into
  // the ring, free after the last block's barrier, and every thread then
  // writes whole 8-column chunks with 16-byte stores (stores of single
  // elements from the accumulator layout were the kernel's largest fixed
  // cost).  When all rows do not fit the ring, two rounds of half the waves.
  constexpr int SR = D + 8, CPR = D / 8, RING = 6 * C::BK * C::LD;
  constexpr int ROWS = C::BQ * SR <= RING ? C::BQ : C::BQ / 2;
  static_assert(ROWS * SR <= RING, "dQ staging must fit the ring");
  e16* stage = &kv_ring[0][0];
#pragma unroll
  for (int round = 0; round < C::BQ / ROWS; ++round) {
    if (w / (ROWS / 32) == round) {
      const int lw = w % (ROWS / 32);
#pragma unroll
      for (int n = 0; n < C::DT; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stage[(32 * lw + 8 * (r >> 2) + 4 * g + (r & 3)) * SR + 32 * n + c] =
              (e16)(dq_acc[n][r] * (DROP ? a.sm_scale * a.m.keep_scale : a.sm_scale));
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < ROWS * CPR / C::NT; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / CPR, col = (chunk % CPR) * 8;
      const int qr = q0 + round * ROWS + row;
      if (qr < NQ) store8(at<e16>(a.dq, b, h, qr) + col, *(const e16x8*)(stage + row * SR + col));
    }
    if (round + 1 < C::BQ / ROWS) __syncthreads();
  }
}

template <int D, bool DROP>
__global__ void __launch_bounds__(QCfg<D>::NT, QCfg<D>::MINB) dq_kernel(BwdArgs a) {
  int bh, blk;
  wg_coords(a.m.cu_q != nullptr, bh, blk);
  dq_body<D, DROP, QCfg<D>::NT>(a, bh, blk);
}

// Small fixed-length problems with d = 64: the KV-outer and the Q-outer
// workgroups of the deterministic backward in one launch (rows y < nkv are
// KV blocks, the rest query blocks of 256).  The two parts share only
// read-only inputs, so when each alone would leave most of the chip idle
// they run side by side instead of one after the other.  Both parts' LDS
// fits one workgroup only for d = 64.
template <int D, bool DROP>
__global__ void __launch_bounds__(512) bwd_small_kernel(BwdArgs a, int nkv) {
  static_assert(D == 64, "the two parts' LDS fits one workgroup only for d = 64");
  if ((int)blockIdx.y < nkv) dkdv_q2_body<D, DROP>(a, blockIdx.x, blockIdx.y);
  else dq_body<D, DROP, 512>(a, blockIdx.x, blockIdx.y - nkv);
}

// Workgroups the small-problem launch may have: one per CU of an MI355X, so
// that all of them are resident at once (one workgroup fits a CU).
constexpr int kSmallGrid = 256;

template <int D>
hipError_t launch_d(const BwdArgs& a, bool deterministic, hipStream_t s) {
  const int bh = a.B * a.H;
  const bool varlen = a.m.cu_q != nullptr;
  const dim3 grid_kv(bh, grid_blocks(bh, a.m.nk, KvCfg<D>::BC, varlen));
  if constexpr (D == 64) {
    const int nkv = (a.m.nk + KvQCfg<D>::BC - 1) / KvQCfg<D>::BC;
    const int nq = (a.m.nq + QCfg<D, 512>::BQ - 1) / QCfg<D, 512>::BQ;
    if (deterministic && !varlen && (int64_t)bh * (nkv + nq) <= kSmallGrid) {
      hipLaunchKernelGGL(a.m.dropout ? (bwd_small_kernel<D, true>) : (bwd_small_kernel<D, false>),
                         dim3(bh, nkv + nq), dim3(512), 0, s, a, nkv);
      return hipGetLastError();
    }
  }
  if (deterministic) {
    if constexpr (D == 128) {
      const hipError_t e = ::fa::FA_ELEM_NS launch_kv128(a, s);  // qualified: BwdArgs brings fa:: in by ADL
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(a.m.dropout ? (dkdv_q2_kernel<D, true>) : (dkdv_q2_kernel<D, false>), grid_kv,
                         dim3(512), 0, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const dim3 grid_q(bh, grid_blocks(bh, a.m.nq, QCfg<D>::BQ, varlen));
    hipLaunchKernelGGL(a.m.dropout ? (dq_kernel<D, true>) : (dq_kernel<D, false>), grid_q, dim3(QCfg<D>::NT),
                       0, s, a);
  } else {
    hipLaunchKernelGGL((dkdv_atomic_kernel<D>), grid_kv, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd16(const BwdArgs& a, bool deterministic, hipStream_t s) {
  return a.d == 128 ? launch_d<128>(a, deterministic, s) : launch_d<64>(a, deterministic, s);
}

FA_ELEM_NS_END
}  // namespace fa
