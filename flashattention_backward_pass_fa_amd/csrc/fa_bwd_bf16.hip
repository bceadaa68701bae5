// fa_bwd_bf16.hip - bf16 FlashAttention backward for gfx950 (MFMA 32x32x16).
//
// Two kernels ("FlashAttention backward", section "The loop structure"):
//
//  dkdv_kernel  KV-outer: one workgroup owns 128 keys (32 per wave) of one
//               (b, h) and loops over the query blocks that can see them.
//               For each 64-query block it recomputes S = Q K^T and
//               dP = dO V^T on MFMA, rebuilds P = exp(S - L) from the saved
//               LSE ("Lecture 7", "The recomputation trick"), forms
//               dS = P * (dP - D) with the pre-pass scalar D, and
//               accumulates dV += P~^T dO and dK += dS^T Q in fp32
//               registers, written once at the end.  In atomic mode it also
//               adds dS K into an fp32 dQ accumulator with device atomics.
//  dq_kernel    Q-outer: one workgroup owns 128 queries (32 per wave) and
//               loops over the visible key blocks, recomputing S, P, dP, dS
//               to accumulate dQ = dS K in registers: the deterministic,
//               atomic-free dQ.
//
// Layout in LDS: Q, dO (and K, V in dq_kernel) tiles are row-major bf16 with
// a 16-element pad per row.  The k-inside-lane operands of the dV/dK/dQ
// products are read from those same tiles with ds_read_tr16_b64, so no
// transposed copies are kept.  K and V of the wave's own keys live in
// registers for the whole kernel (B operand of S and dP).
// Blocks that are fully masked (causal/window) are never visited; a wave
// whose 64x32 sub-tile is fully masked skips its products; only tiles that
// straddle a mask edge or the sequence end evaluate the per-element mask.

#include "fa_kernels.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct KvCfg {
  static constexpr int BC = 128;          // keys per workgroup
  static constexpr int BR = 64;           // queries per inner iteration
  static constexpr int NT = 256;          // threads (4 waves)
  static constexpr int LD = D + 16;       // LDS row stride of Q/dO/K tiles
  static constexpr int LDS_T = BR + 16;   // LDS row stride of the dS^T tile
  static constexpr int KT = D / 16;       // MFMA k-steps over d
  static constexpr int DT = D / 32;       // 32-wide tiles over d
  static constexpr int CH = D / 8;        // 16-byte chunks per row
  static constexpr int LOADS = BR * CH / NT;
};

template <int D>
struct QCfg {
  static constexpr int BQ = 128;          // queries per workgroup
  static constexpr int BK = 64;           // keys per inner iteration
  static constexpr int NT = 256;
  static constexpr int LD = D + 16;
  static constexpr int KT = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BK * CH / NT;
};

__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ void store8(bf16* p, bf16x8 v) { *(bf16x8*)p = v; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
  return z;
}

// Is every (query, key) of rows [q0, q0+nq) x keys [k0, k0+nk) visible?
__device__ __forceinline__ bool block_full(const MaskArgs& m, int q0, int nq, int k0, int nk) {
  bool ok = (q0 + nq <= m.n) & (k0 + nk <= m.n);
  if (m.causal) ok &= (k0 + nk - 1 <= q0);
  if (m.wl >= 0) ok &= (k0 >= q0 + nq - 1 - m.wl);
  if (m.wr >= 0) ok &= (k0 + nk - 1 <= q0 + m.wr);
  return ok;
}

// Is every (query, key) of that block hidden?
__device__ __forceinline__ bool block_dead(const MaskArgs& m, int q0, int nq, int k0, int nk) {
  bool dead = (q0 >= m.n) | (k0 >= m.n);
  if (m.causal) dead |= (k0 > q0 + nq - 1);
  if (m.wl >= 0) dead |= (k0 + nk - 1 < q0 - m.wl);
  if (m.wr >= 0) dead |= (k0 > q0 + nq - 1 + m.wr);
  return dead;
}

// ---------------------------------------------------------------- KV-outer

template <int D, bool ATOMIC>
__global__ void __launch_bounds__(256, 1) dkdv_kernel(BwdArgs a) {
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 sQ[2][C::BR * C::LD];
  __shared__ __attribute__((aligned(16))) bf16 sO[2][C::BR * C::LD];
  __shared__ __attribute__((aligned(16))) bf16 sK[ATOMIC ? C::BC * C::LD : 8];
  __shared__ __attribute__((aligned(16))) bf16 sT[ATOMIC ? C::BC * C::LDS_T : 8];
  __shared__ __attribute__((aligned(16))) float sL[2][C::BR];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.m.n;
  const int kv0 = blockIdx.y * C::BC;
  const int kvw = kv0 + 32 * w;

  // Query rows that can see at least one of the block's keys.
  int q_lo = 0, q_hi = N;
  if (a.m.causal) q_lo = max(q_lo, kv0);
  if (a.m.wr >= 0) q_lo = max(q_lo, kv0 - a.m.wr);
  if (a.m.wl >= 0) q_hi = min(q_hi, kv0 + C::BC + a.m.wl);
  const int it0 = q_lo / C::BR;
  const int it1 = q_lo < q_hi ? (q_hi + C::BR - 1) / C::BR : it0;

  // This wave's 32 keys: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kreg[C::KT], vreg[C::KT];
  {
    const int row = kvw + c;
    const bool ok = row < N;
    const bf16* kp = at<bf16>(a.k, b, h, ok ? row : 0);
    const bf16* vp = at<bf16>(a.v, b, h, ok ? row : 0);
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
      kreg[t] = ok ? load8(kp + 16 * t + 8 * g) : zero8();
      vreg[t] = ok ? load8(vp + 16 * t + 8 * g) : zero8();
    }
  }
  if (ATOMIC) {
#pragma unroll
    for (int x = 0; x < C::BC * C::CH / C::NT; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int key = kv0 + row;
      store8(sK + row * C::LD + col, key < N ? load8(at<bf16>(a.k, b, h, key) + col) : zero8());
    }
  }

  const int64_t row_base = (int64_t)bh * N;
  bf16x8 pq[C::LOADS], po[C::LOADS];
  float pl = 0.f, pd = 0.f;

  auto load_tile = [&](int it) {
    const int q0 = it * C::BR;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int qr = q0 + row;
      if (qr < N) {
        pq[x] = load8(at<bf16>(a.q, b, h, qr) + col);
        po[x] = load8(at<bf16>(a.dout, b, h, qr) + col);
      } else {
        pq[x] = zero8();
        po[x] = zero8();
      }
    }
    if (tid < C::BR) {
      const int qr = q0 + tid;
      pl = qr < N ? a.lse[row_base + qr] * kLog2e : 0.f;
      pd = qr < N ? a.delta[row_base + qr] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      store8(&sQ[buf][row * C::LD + col], pq[x]);
      store8(&sO[buf][row * C::LD + col], po[x]);
    }
    if (tid < C::BR) {
      sL[buf][tid] = pl;
      sD[buf][tid] = pd;
    }
  };

  f32x16 dk_acc[C::DT], dv_acc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) {
    dk_acc[n] = f32x16{};
    dv_acc[n] = f32x16{};
  }

  if (it0 < it1) {
    load_tile(it0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = it0; it < it1; ++it) {
    const int buf = (it - it0) & 1;
    const bool has_next = it + 1 < it1;
    if (has_next) load_tile(it + 1);
    const bf16* Qs = sQ[buf];
    const bf16* Os = sO[buf];
    const int q0 = it * C::BR;
    const bool dead = block_dead(a.m, q0, C::BR, kvw, 32);
    const bool full = block_full(a.m, q0, C::BR, kvw, 32);

    bf16x8 pa[4], da[4];  // A operands (16-query k-steps) of dV and dK
    if (!dead) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[qt] = f32x16{};
        dp[qt] = f32x16{};
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
          const bf16x8 aq = load8(Qs + (32 * qt + c) * C::LD + 16 * t + 8 * g);
          const bf16x8 ao = load8(Os + (32 * qt + c) * C::LD + 16 * t + 8 * g);
          s[qt] = mfma32x32x16(aq, kreg[t], s[qt]);
          dp[qt] = mfma32x32x16(ao, vreg[t], dp[qt]);
        }
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * qt + 8 * (r >> 2) + 4 * g + (r & 3);
          const float l2 = sL[buf][ql];
          const float dd = sD[buf][ql];
          float p = fast_exp2(s[qt][r] * a.scale_log2 - l2);
          float dpv = dp[qt][r];
          if (!full && !visible(a.m, q0 + ql, kvw + c)) p = 0.f;
          float pdrop = p;
          if (a.m.dropout) {
            const bool keep = dropout_keep(a.m, b, h, q0 + ql, kvw + c);
            pdrop = keep ? p * a.m.keep_scale : 0.f;
            dpv = keep ? dpv * a.m.keep_scale : 0.f;
          }
          const float ds = p * (dpv - dd);
          pa[2 * qt + (r >> 3)][r & 7] = (bf16)pdrop;
          da[2 * qt + (r >> 3)][r & 7] = (bf16)ds;
        }
      }
#pragma unroll
      for (int n = 0; n < C::DT; ++n) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 bo = tr_operand(Os, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
          const bf16x8 bq = tr_operand(Qs, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
          dv_acc[n] = mfma32x32x16(pa[u], bo, dv_acc[n]);
          dk_acc[n] = mfma32x32x16(da[u], bq, dk_acc[n]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) da[u] = zero8();
    }

    if (ATOMIC) {
      // dS^T of this wave's keys into LDS: sT[key][query].
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bf16x8 src = da[2 * qt + (rr >> 1)];
          const int s0 = (rr & 1) * 4;
          const bf16x4 v4 = {src[s0], src[s0 + 1], src[s0 + 2], src[s0 + 3]};
          *(bf16x4*)(sT + (32 * w + c) * C::LDS_T + 32 * qt + 8 * rr + 4 * g) = v4;
        }
      }
      __syncthreads();
      // dQ partial of the 64 queries over the block's 128 keys.
      constexpr int MT = D == 128 ? 2 : 1;  // 32-query tiles per wave
      const int nt = D == 128 ? w : (w & 1);
      const int mt0 = D == 128 ? 0 : (w >> 1);
      f32x16 dq[MT];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) dq[mi] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::BC / 16; ++t) {
        const bf16x8 bk = tr_operand(sK, C::LD, 16 * t + 8 * g, 16 * t + 8 * g + 4, 32 * nt, lane);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          const bf16x8 as =
              tr_operand(sT, C::LDS_T, 16 * t + 8 * g, 16 * t + 8 * g + 4, 32 * (mt0 + mi), lane);
          dq[mi] = mfma32x32x16(as, bk, dq[mi]);
        }
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = q0 + 32 * (mt0 + mi) + 8 * (r >> 2) + 4 * g + (r & 3);
          if (qr < N) unsafeAtomicAdd(a.dq_acc + (row_base + qr) * D + 32 * nt + c, dq[mi][r]);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // dK = sm_scale * dS^T Q, dV = P~^T dO: one rounding to bf16 at the store.
#pragma unroll
  for (int n = 0; n < C::DT; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kvw + 8 * (r >> 2) + 4 * g + (r & 3);
      if (key < N) {
        at<bf16>(a.dk, b, h, key)[32 * n + c] = (bf16)(dk_acc[n][r] * a.sm_scale);
        at<bf16>(a.dv, b, h, key)[32 * n + c] = (bf16)(dv_acc[n][r]);
      }
    }
  }
}

// ---------------------------------------------------------------- Q-outer

template <int D>
__global__ void __launch_bounds__(256, 1) dq_kernel(BwdArgs a) {
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][C::BK * C::LD];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][C::BK * C::LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int N = a.m.n;
  const int q0 = blockIdx.y * C::BQ;
  const int qw = q0 + 32 * w;
  const int myq = qw + c;
  const int64_t row_base = (int64_t)bh * N;

  // This wave's 32 queries: B operands of S^T = K Q^T and dP^T = V dO^T.
  bf16x8 qreg[C::KT], oreg[C::KT];
  {
    const bool ok = myq < N;
    const bf16* qp = at<bf16>(a.q, b, h, ok ? myq : 0);
    const bf16* op = at<bf16>(a.dout, b, h, ok ? myq : 0);
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
      qreg[t] = ok ? load8(qp + 16 * t + 8 * g) : zero8();
      oreg[t] = ok ? load8(op + 16 * t + 8 * g) : zero8();
    }
  }
  const float l2 = myq < N ? a.lse[row_base + myq] * kLog2e : 0.f;
  const float dd = myq < N ? a.delta[row_base + myq] : 0.f;

  int k_lo = 0, k_hi = N;
  if (a.m.causal) k_hi = min(k_hi, q0 + C::BQ);
  if (a.m.wl >= 0) k_lo = max(k_lo, q0 - a.m.wl);
  if (a.m.wr >= 0) k_hi = min(k_hi, q0 + C::BQ + a.m.wr);
  const int jt0 = k_lo / C::BK;
  const int jt1 = k_lo < k_hi ? (k_hi + C::BK - 1) / C::BK : jt0;

  bf16x8 pk[C::LOADS], pv[C::LOADS];
  auto load_tile = [&](int jt) {
    const int k0 = jt * C::BK;
#pragma unroll
    for (int x = 0; x < C::LOADS; ++x) {
      const int chunk = tid + x * C::NT;
      const int row = chunk / C::CH, col = (chunk % C::CH) * 8;
      const int kr = k0 + row;
      if (kr < N) {
        pk[x] = load8(at<bf16>(a.k, b, h, kr) + col);
        pv[x] = load8(at<bf16>(a.v, b, h, kr) + col);
      } else {
        pk[x] = zero8();
        pv[x] = zero8();
      }
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

  f32x16 dq_acc[C::DT];
#pragma unroll
  for (int n = 0; n < C::DT; ++n) dq_acc[n] = f32x16{};

  if (jt0 < jt1) {
    load_tile(jt0);
    store_tile(0);
  }
  __syncthreads();

  for (int jt = jt0; jt < jt1; ++jt) {
    const int buf = (jt - jt0) & 1;
    const bool has_next = jt + 1 < jt1;
    if (has_next) load_tile(jt + 1);
    const bf16* Ks = sK[buf];
    const bf16* Vs = sV[buf];
    const int k0 = jt * C::BK;
    const bool dead = block_dead(a.m, qw, 32, k0, C::BK);
    const bool full = block_full(a.m, qw, 32, k0, C::BK);
    if (!dead) {
      f32x16 st[2], dpt[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        st[kt] = f32x16{};
        dpt[kt] = f32x16{};
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
          const bf16x8 ak = load8(Ks + (32 * kt + c) * C::LD + 16 * t + 8 * g);
          const bf16x8 av = load8(Vs + (32 * kt + c) * C::LD + 16 * t + 8 * g);
          st[kt] = mfma32x32x16(ak, qreg[t], st[kt]);
          dpt[kt] = mfma32x32x16(av, oreg[t], dpt[kt]);
        }
      }
      bf16x8 da[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
          float p = fast_exp2(st[kt][r] * a.scale_log2 - l2);
          float dpv = dpt[kt][r];
          if (!full && !visible(a.m, myq, key)) p = 0.f;
          if (a.m.dropout) {
            const bool keep = dropout_keep(a.m, b, h, myq, key);
            dpv = keep ? dpv * a.m.keep_scale : 0.f;
          }
          da[2 * kt + (r >> 3)][r & 7] = (bf16)(p * (dpv - dd));
        }
      }
#pragma unroll
      for (int n = 0; n < C::DT; ++n) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 bk = tr_operand(Ks, C::LD, 16 * u + 4 * g, 16 * u + 8 + 4 * g, 32 * n, lane);
          dq_acc[n] = mfma32x32x16(da[u], bk, dq_acc[n]);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int n = 0; n < C::DT; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = qw + 8 * (r >> 2) + 4 * g + (r & 3);
      if (qr < N) at<bf16>(a.dq, b, h, qr)[32 * n + c] = (bf16)(dq_acc[n][r] * a.sm_scale);
    }
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, bool deterministic, hipStream_t s) {
  const int bh = a.B * a.H;
  const dim3 grid_kv(bh, (a.m.n + KvCfg<D>::BC - 1) / KvCfg<D>::BC);
  if (deterministic) {
    hipLaunchKernelGGL((dkdv_kernel<D, false>), grid_kv, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid_q(bh, (a.m.n + QCfg<D>::BQ - 1) / QCfg<D>::BQ);
    hipLaunchKernelGGL((dq_kernel<D>), grid_q, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((dkdv_kernel<D, true>), grid_kv, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, bool deterministic, hipStream_t s) {
  return a.d == 128 ? launch_d<128>(a, deterministic, s) : launch_d<64>(a, deterministic, s);
}

}  // namespace fa
