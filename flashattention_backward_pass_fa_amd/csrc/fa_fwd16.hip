// fa_fwd16.hip - 16-bit (bf16 or fp16) FlashAttention forward for gfx950,
// emitting O and L.  Compiled once per element type (see fa_device.h).
//
// "FlashAttention backward", section "What the forward left behind": the
// forward keeps only O and the per-row log-sum-exp L_i = m_i + log l_i.
// One workgroup owns 32 queries per wave of one (b, h) and streams
// 64-key blocks through LDS (the shape per head dim is set by FCfg).  Each wave computes S^T = K Q^T so that its
// lanes index queries: the running max m and sum l of the online softmax
// are then per-lane scalars (one exchange with the other lane half per
// block), and O^T += V^T P~^T keeps the query index across lanes too, so the
// per-row rescale is a per-lane multiply.  Dropout zeroes the dropped
// weights that feed O (never the normaliser l); the kept ones enter the
// 16-bit product unscaled and 1 / (1 - p) joins 1 / l at the end, so the
// weight of a row's largest score (exactly 1) is not rounded.

#include <type_traits>

#include "fa_kernels.h"

namespace fa {
FA_ELEM_NS_BEGIN
namespace {

constexpr float kLn2 = 0.6931471805599453f;

// d = 128: one workgroup of 8 waves per CU, K/V in a ring of three blocks
// (the scores of the next block are formed beside the softmax of this one);
// d = 64: three workgroups of 4 waves per CU (at most 168 registers, three
// waves per SIMD), K/V double-buffered, one block at a time (measured faster
// there: independent workgroups overlap the Philox rounds of one with the
// others' products).
template <int D>
struct FCfg {
  static constexpr int NT = D == 128 ? 512 : 256;  // 32 queries per wave
  static constexpr int MINB = D == 128 ? 1 : 3;    // workgroups per CU
  static constexpr int RING = D == 128 ? 3 : 2;    // K/V blocks in LDS
  static constexpr int BQ = NT / 2;                // queries per workgroup
  static constexpr int BK = 64;        // keys per block
  static constexpr int LD = lds_stride(D);
  static constexpr int KT = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BK * CH / NT;  // 16-byte chunks per thread per K (and V) block
};

__device__ __forceinline__ e16x8 load8(const e16* p) { return *(const e16x8*)p; }
__device__ __forceinline__ void store8(e16* p, e16x8 v) { *(e16x8*)p = v; }

template <int D, bool DROP>
__global__ void __launch_bounds__(FCfg<D>::NT, FCfg<D>::MINB) fwd_kernel(FwdArgs a) {
  using C = FCfg<D>;
  __shared__ __attribute__((aligned(16))) e16 sK[C::RING][C::BK * C::LD];
  __shared__ __attribute__((aligned(16))) e16 sV[C::RING][C::BK * C::LD];

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave: keep it (and all derived from it) scalar
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), c = lane & 31, g = lane >> 5;
  int bh, blk;
  wg_coords(a.m.cu_q != nullptr, bh, blk);
  const int b = bh / a.H, h = bh - b * a.H;
  {
    const SeqRows r = seq_localize(a.m, b);
    if (a.m.cu_q) {
      shift_rows<e16>(a.q, r.q0);
      shift_rows<e16>(a.o, r.q0);
      shift_rows<e16>(a.k, r.k0);
      shift_rows<e16>(a.v, r.k0);
    }
  }
  const int NQ = a.m.nq, NK = a.m.nk;
  // Longest first: with a causal mask the last query blocks see the most keys.
  const int nblk = (NQ + C::BQ - 1) / C::BQ;
  if (blk >= nblk) return;  // past this sequence's queries
  const int q0 = (a.m.causal ? nblk - 1 - blk : blk) * C::BQ;
  const int qw = q0 + 32 * w;
  const int myq = qw + c;

  // Rows past the end are read as copies of the last row (a clamped index):
  // a load under a condition compiles to a branch that waits for it.  The
  // copies are finite; query copies only feed O rows that are never stored,
  // key copies are masked.
  e16x8 qreg[C::KT];
  {
    const e16* qp = at<e16>(a.q, b, h, min(myq, NQ - 1));
#pragma unroll
    for (int t = 0; t < C::KT; ++t) qreg[t] = load8(qp + 16 * t + 8 * g);
  }

  // Keys that at least one of the block's queries can see (workgroup-uniform;
  // saying so keeps the loop bounds in scalar registers).
  const int k_lo = __builtin_amdgcn_readfirstlane(max(0, q0 - a.m.lo_off));
  const int k_hi = __builtin_amdgcn_readfirstlane(min(NK, q0 + C::BQ + a.m.hi_off));
  const int jt0 = k_lo / C::BK;
  const int jt1 = k_lo < k_hi ? (k_hi + C::BK - 1) / C::BK : jt0;

  e16x8 pk[C::LOADS], pv[C::LOADS];
  auto load_into = [&](int jt, e16x8* kd, e16x8* vd) {
    const int k0 = jt * C::BK;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int kc = min(k0 + row, NK - 1);
      kd[x] = load8(at<e16>(a.k, b, h, kc) + col);
      vd[x] = load8(at<e16>(a.v, b, h, kc) + col);
    }
  };
  auto store_from = [&](int buf, const e16x8* ks, const e16x8* vs) {
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(&sK[buf][row * C::LD + col], ks[x]);
      store8(&sV[buf][row * C::LD + col], vs[x]);
    }
  };
  auto ring = [&](int jt) { return C::RING == 3 ? (jt - jt0) % 3 : (jt - jt0) & 1; };
  // Three buffers: the start of every iteration publishes block jt + 2,
  // whose loads were issued one iteration earlier (its buffer held block
  // jt - 1, free since the last barrier; it is first read after this
  // iteration's barrier), and issues block jt + 3's loads.  Two buffers:
  // block jt + 1 is loaded at the start and published at the end.
  auto prefetch = [&](int jt) {
    if (C::RING == 3) {
      if (jt + 2 < jt1) store_from(ring(jt + 2), pk, pv);
      if (jt + 3 < jt1) load_into(jt + 3, pk, pv);
    } else if (jt + 1 < jt1) {
      load_into(jt + 1, pk, pv);
    }
  };
  auto finish_block = [&](int jt) {
    if (C::RING == 2 && jt + 1 < jt1) store_from(ring(jt + 1), pk, pv);
    lds_barrier();
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) oacc[n] = f32x16{};
  float m_run = -INFINITY;  // running max of the log2-scaled scores
  float l_run = 0.f;        // this lane half's share of the normaliser

  if (jt0 < jt1) {
    e16x8 k0[C::LOADS], v0[C::LOADS], k1[C::LOADS], v1[C::LOADS];
    load_into(jt0, k0, v0);
    if (C::RING == 3 && jt0 + 1 < jt1) load_into(jt0 + 1, k1, v1);
    if (C::RING == 3 && jt0 + 2 < jt1) load_into(jt0 + 2, pk, pv);
    store_from(0, k0, v0);
    if (C::RING == 3 && jt0 + 1 < jt1) store_from(1, k1, v1);
  }
  __syncthreads();

  // S^T = K Q^T of one 64-key block (two 32-key halves), log2-scaled
  auto scores = [&](int buf, f32x16 (&st)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::KT; ++t)
        st[kt] = mfma32x32x16(load8(&sK[buf][(32 * kt + c) * C::LD + 16 * t + 8 * g]), qreg[t], st[kt]);
    }
  };
  // Online softmax of one block: MASKED evaluates the element mask.  Leaves
  // the 16-bit weights P~^T (B operands of O^T += V^T P~^T) in pb.
  auto softmax = [&](int jt, f32x16 (&st)[2], e16x8 (&pb)[4], auto masked) {
    const int k0 = jt * C::BK;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s2 = st[kt][r] * a.scale_log2;
        if (decltype(masked)::value) {
          const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
          if (!visible(a.m, myq, key)) s2 = -INFINITY;
        }
        st[kt][r] = s2;
        mx = fmaxf(mx, s2);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // rescale only when some lane's running max moved (alpha == 1 otherwise,
    // and a product with 1 changes nothing)
    if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < C::DT; ++n) oacc[n] *= alpha;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // this lane's keys k0 + 32 kt + 8 rr + 4 g + (0..3) at bits 4 rr + (0..3)
      const uint32_t kp = DROP ? dropout_keep_lane(a.m, b, h, myq, k0 + 32 * kt, g) : ~0u;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t keep = (kp >> (4 * rr)) & 0xFu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          const float p = fast_exp2(st[kt][r] - m_use);
          l_run += p;
          float pd = p;
          if (DROP) pd = (keep >> e) & 1u ? p : 0.f;  // 1 / (1 - p) joins 1 / l at the end
          pb[2 * kt + (r >> 3)][r & 7] = (e16)pd;
        }
      }
    }
    m_run = m_new;
  };
  // O^T += V^T P~^T over one block
  auto accumulate = [&](int buf, const e16x8 (&pb)[4]) {
#pragma unroll
    for (int n = 0; n < C::DT; ++n) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const e16x8 av = tr_operand(sV[buf], C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
        oacc[n] = mfma32x32x16(av, pb[u], oacc[n]);
      }
    }
  };
  std::integral_constant<bool, true> masked;
  std::integral_constant<bool, false> unmasked;
  auto general = [&](int jt) {
    prefetch(jt);
    f32x16 st[2];
    e16x8 pb[4];
    scores(ring(jt), st);
    softmax(jt, st, pb, masked);
    accumulate(ring(jt), pb);
    finish_block(jt);
  };
  // Key blocks [jtA, jtB) are seen by all of the block's queries with no
  // mask edge: the first query bounds k0 from above (causality, right
  // window), the last real query from below (left window).  Rows past the
  // sequence end need no mask: their O is never stored.
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
  int jt = jt0;
  for (; jt < jtA; ++jt) general(jt);
  if (DROP || C::RING == 2) {
    // one block at a time, no mask (with dropout the Philox rounds already
    // sit beside the products, and the pipelined form measured slower)
    for (; jt < jtB; ++jt) {
      prefetch(jt);
      f32x16 st[2];
      e16x8 pb[4];
      scores(ring(jt), st);
      softmax(jt, st, pb, unmasked);
      accumulate(ring(jt), pb);
      finish_block(jt);
    }
  } else if (jtA < jtB) {
    // software-pipelined: the scores of block jt + 1 are formed beside the
    // softmax of block jt
    f32x16 st[2];
    scores(ring(jtA), st);
    for (; jt + 1 < jtB; ++jt) {
      prefetch(jt);
      f32x16 stn[2];
      scores(ring(jt + 1), stn);
      e16x8 pb[4];
      softmax(jt, st, pb, unmasked);
      accumulate(ring(jt), pb);
      finish_block(jt);
      st[0] = stn[0];
      st[1] = stn[1];
    }
    prefetch(jt);
    e16x8 pb[4];
    softmax(jt, st, pb, unmasked);
    accumulate(ring(jt), pb);
    finish_block(jt);
    ++jt;
  }
  for (; jt < jt1; ++jt) general(jt);

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (myq < NQ) {
    // a row that sees no key (possible when nq > nk, or through a window)
    // has an empty sum: O = 0 and L = log 0 = -inf
    const float inv = l_tot > 0.f ? (DROP ? a.m.keep_scale / l_tot : 1.0f / l_tot) : 0.f;
    e16* op = at<e16>(a.o, b, h, myq);
#pragma unroll
    for (int n = 0; n < C::DT; ++n) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const e16x4 v4 = {(e16)(oacc[n][4 * rr] * inv), (e16)(oacc[n][4 * rr + 1] * inv),
                           (e16)(oacc[n][4 * rr + 2] * inv), (e16)(oacc[n][4 * rr + 3] * inv)};
        *(e16x4*)(op + 32 * n + 8 * rr + 4 * g) = v4;
      }
    }
    if (g == 0) a.lse[(int64_t)bh * a.ln + myq] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd16(const FwdArgs& a, hipStream_t s) {
  const int bh = a.B * a.H;
  const bool varlen = a.m.cu_q != nullptr;
  if (a.d == 128)
    hipLaunchKernelGGL(a.m.dropout ? (fwd_kernel<128, true>) : (fwd_kernel<128, false>),
                       dim3(bh, grid_blocks(bh, a.m.nq, FCfg<128>::BQ, varlen)), dim3(FCfg<128>::NT), 0, s, a);
  else
    hipLaunchKernelGGL(a.m.dropout ? (fwd_kernel<64, true>) : (fwd_kernel<64, false>),
                       dim3(bh, grid_blocks(bh, a.m.nq, FCfg<64>::BQ, varlen)), dim3(FCfg<64>::NT), 0, s, a);
  return hipGetLastError();
}

FA_ELEM_NS_END
}  // namespace fa
