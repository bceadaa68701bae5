// fa_fwd16.hip - 16-bit (bf16 or fp16) FlashAttention forward for gfx950,
// emitting O and L.  Compiled once per element type (see fa_device.h).
//
// "FlashAttention backward", section "What the forward left behind": the
// forward keeps only O and the per-row log-sum-exp L_i = m_i + log l_i.
// One workgroup owns 128 queries (32 per wave) of one (b, h) and streams
// 64-key blocks through LDS.  Each wave computes S^T = K Q^T so that its
// lanes index queries: the running max m and sum l of the online softmax
// are then per-lane scalars (one exchange with the other lane half per
// block), and O^T += V^T P~^T keeps the query index across lanes too, so the
// per-row rescale is a per-lane multiply.  Dropout multiplies the weights
// that feed O but not the normaliser l.

#include <type_traits>

#include "fa_kernels.h"

namespace fa {
FA_ELEM_NS_BEGIN
namespace {

constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct FCfg {
  static constexpr int BQ = 128;
  static constexpr int BK = 64;
  static constexpr int NT = 256;
  static constexpr int LD = lds_stride(D);
  static constexpr int KT = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BK * CH / NT;
};

__device__ __forceinline__ e16x8 load8(const e16* p) { return *(const e16x8*)p; }
__device__ __forceinline__ void store8(e16* p, e16x8 v) { *(e16x8*)p = v; }

template <int D, bool DROP>
__global__ void __launch_bounds__(256, 2) fwd_kernel(FwdArgs a) {
  using C = FCfg<D>;
  __shared__ __attribute__((aligned(16))) e16 sK[2][C::BK * C::LD];
  __shared__ __attribute__((aligned(16))) e16 sV[2][C::BK * C::LD];

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
  auto load_tile = [&](int jt) {
    const int k0 = jt * C::BK;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int kc = min(k0 + row, NK - 1);
      pk[x] = load8(at<e16>(a.k, b, h, kc) + col);
      pv[x] = load8(at<e16>(a.v, b, h, kc) + col);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(&sK[buf][row * C::LD + col], pk[x]);
      store8(&sV[buf][row * C::LD + col], pv[x]);
    }
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) oacc[n] = f32x16{};
  float m_run = -INFINITY;  // running max of the log2-scaled scores
  float l_run = 0.f;        // this lane half's share of the normaliser

  if (jt0 < jt1) {
    load_tile(jt0);
    store_tile(0);
  }
  __syncthreads();

  // One 64-key block.  FULL: every (query, key) of the workgroup's block is
  // visible, so no element mask is evaluated.
  auto step = [&](int jt, auto full) {
    const int buf = (jt - jt0) & 1;
    const bool has_next = jt + 1 < jt1;
    if (has_next) load_tile(jt + 1);
    const e16* Ks = sK[buf];
    const e16* Vs = sV[buf];
    const int k0 = jt * C::BK;

    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::KT; ++t) {
        const e16x8 ak = load8(Ks + (32 * kt + c) * C::LD + 16 * t + 8 * g);
        st[kt] = mfma32x32x16(ak, qreg[t], st[kt]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s2 = st[kt][r] * a.scale_log2;
        if (!decltype(full)::value) {
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
    e16x8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        // keys j4 .. j4 + 3 of this lane's query share one dropout block
        const uint32_t keep = DROP ? dropout_keep4(a.m, b, h, myq, k0 + 32 * kt + 8 * rr + 4 * g) : 0xFu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          const float p = fast_exp2(st[kt][r] - m_use);
          l_run += p;
          float pd = p;
          if (DROP) pd = (keep >> e) & 1u ? p * a.m.keep_scale : 0.f;
          pb[2 * kt + (r >> 3)][r & 7] = (e16)pd;
        }
      }
    }
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < C::DT; ++n) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const e16x8 av = tr_operand(Vs, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
        oacc[n] = mfma32x32x16(av, pb[u], oacc[n]);
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
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
  std::integral_constant<bool, false> general;
  std::integral_constant<bool, true> fast;
  int jt = jt0;
  for (; jt < jtA; ++jt) step(jt, general);
  for (; jt < jtB; ++jt) step(jt, fast);
  for (; jt < jt1; ++jt) step(jt, general);

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (myq < NQ) {
    // a row that sees no key (possible when nq > nk, or through a window)
    // has an empty sum: O = 0 and L = log 0 = -inf
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
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
  const dim3 grid(a.B * a.H, grid_blocks(a.B * a.H, a.m.nq, 128, a.m.cu_q != nullptr));
  if (a.d == 128)
    hipLaunchKernelGGL(a.m.dropout ? (fwd_kernel<128, true>) : (fwd_kernel<128, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(a.m.dropout ? (fwd_kernel<64, true>) : (fwd_kernel<64, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

FA_ELEM_NS_END
}  // namespace fa
