// fa_f32.hip - fp32 forward and backward (one thread per output row).
//
// The fp32 path serves small fp32 problems at full fp32 accuracy; it is
// written for clarity, not speed (bf16 is the MFMA path).  The formulas are
// the same as the bf16 kernels: P_ij = exp(S_ij - L_i) recomputed from the
// saved LSE, dS = P * (dP - D), dV = P~^T dO, dK = sm_scale dS^T Q,
// dQ = sm_scale dS K ("Lecture 7", "The math"; "FlashAttention backward",
// "The gradients, and the one scalar that makes them local").  dQ always
// comes from the Q-outer kernel, so the fp32 path is deterministic in both
// modes and never touches the dQ workspace.

#include "fa_kernels.h"

namespace fa {
namespace {

// Visible key range [lo, hi) of query row i (empty when hi <= lo).
__device__ __forceinline__ void key_range(const MaskArgs& m, int i, int& lo, int& hi) {
  lo = max(0, i - m.lo_off);
  hi = min(m.nk, i + m.hi_off + 1);
}

// Query range [lo, hi) that sees key row j.
__device__ __forceinline__ void query_range(const MaskArgs& m, int j, int& lo, int& hi) {
  lo = max(0, j - m.hi_off);
  hi = min(m.nq, j + m.lo_off + 1);
}

// Specialise a call to sequence b: lengths, mask offsets, packed rows.
__device__ __forceinline__ void localize(FwdArgs& a, int b) {
  const SeqRows r = seq_localize(a.m, b);
  if (a.m.cu_q) {
    shift_rows<float>(a.q, r.q0);
    shift_rows<float>(a.o, r.q0);
    shift_rows<float>(a.k, r.k0);
    shift_rows<float>(a.v, r.k0);
  }
}

__device__ __forceinline__ void localize(BwdArgs& a, int b) {
  const SeqRows r = seq_localize(a.m, b);
  if (a.m.cu_q) {
    shift_rows<float>(a.q, r.q0);
    shift_rows<float>(a.dout, r.q0);
    shift_rows<float>(a.dq, r.q0);
    shift_rows<float>(a.k, r.k0);
    shift_rows<float>(a.v, r.k0);
    shift_rows<float>(a.dk, r.k0);
    shift_rows<float>(a.dv, r.k0);
  }
}

template <int DM>
__global__ void __launch_bounds__(64) fwd_f32_kernel(FwdArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H;
  localize(a, b);
  const int i = blockIdx.y * 64 + threadIdx.x;
  const int d = a.d;
  if (i >= a.m.nq) return;
  const float scale = a.sm_scale;
  float q[DM], o[DM];
  const float* qp = at<float>(a.q, b, h, i);
#pragma unroll
  for (int c = 0; c < DM; ++c) {
    q[c] = c < d ? qp[c] : 0.f;
    o[c] = 0.f;
  }
  int lo, hi;
  key_range(a.m, i, lo, hi);
  float m_run = -INFINITY, l_run = 0.f;
  for (int j = lo; j < hi; ++j) {
    const float* kp = at<float>(a.k, b, h, j);
    const float* vp = at<float>(a.v, b, h, j);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < DM; ++c)
      if (c < d) s = fmaf(q[c], kp[c], s);
    s *= scale;
    const float m_new = fmaxf(m_run, s);
    const float alpha = expf(m_run - m_new);
    const float p = expf(s - m_new);
    l_run = l_run * alpha + p;
    float pd = p;
    if (a.m.dropout) pd = dropout_keep(a.m, b, h, i, j) ? p * a.m.keep_scale : 0.f;
#pragma unroll
    for (int c = 0; c < DM; ++c)
      if (c < d) o[c] = fmaf(pd, vp[c], o[c] * alpha);
    m_run = m_new;
  }
  // a row that sees no key has an empty sum: O = 0 and L = log 0 = -inf
  float* op = at<float>(a.o, b, h, i);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int c = 0; c < DM; ++c)
    if (c < d) op[c] = o[c] * inv;
  a.lse[(int64_t)bh * a.ln + i] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

template <int DM>
__global__ void __launch_bounds__(64) dkdv_f32_kernel(BwdArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H;
  localize(a, b);
  const int j = blockIdx.y * 64 + threadIdx.x;
  const int d = a.d;
  if (j >= a.m.nk) return;
  const int64_t row_base = (int64_t)bh * a.ln;
  float kj[DM], vj[DM], dk[DM], dv[DM];
  const float* kp = at<float>(a.k, b, h, j);
  const float* vp = at<float>(a.v, b, h, j);
#pragma unroll
  for (int c = 0; c < DM; ++c) {
    kj[c] = c < d ? kp[c] : 0.f;
    vj[c] = c < d ? vp[c] : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  int lo, hi;
  query_range(a.m, j, lo, hi);
  for (int i = lo; i < hi; ++i) {
    const float* qp = at<float>(a.q, b, h, i);
    const float* gp = at<float>(a.dout, b, h, i);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < DM; ++c)
      if (c < d) {
        s = fmaf(qp[c], kj[c], s);
        dp = fmaf(gp[c], vj[c], dp);
      }
    const float p = expf(s * a.sm_scale - a.lse[row_base + i]);
    float pd = p;
    if (a.m.dropout) {
      const bool keep = dropout_keep(a.m, b, h, i, j);
      pd = keep ? p * a.m.keep_scale : 0.f;
      dp = keep ? dp * a.m.keep_scale : 0.f;
    }
    const float ds = p * (dp - a.delta[row_base + i]);
#pragma unroll
    for (int c = 0; c < DM; ++c)
      if (c < d) {
        dv[c] = fmaf(pd, gp[c], dv[c]);
        dk[c] = fmaf(ds, qp[c], dk[c]);
      }
  }
  float* dkp = at<float>(a.dk, b, h, j);
  float* dvp = at<float>(a.dv, b, h, j);
#pragma unroll
  for (int c = 0; c < DM; ++c)
    if (c < d) {
      dkp[c] = dk[c] * a.sm_scale;
      dvp[c] = dv[c];
    }
}

template <int DM>
__global__ void __launch_bounds__(64) dq_f32_kernel(BwdArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H;
  localize(a, b);
  const int i = blockIdx.y * 64 + threadIdx.x;
  const int d = a.d;
  if (i >= a.m.nq) return;
  const int64_t row_base = (int64_t)bh * a.ln;
  float qi[DM], gi[DM], dq[DM];
  const float* qp = at<float>(a.q, b, h, i);
  const float* gp = at<float>(a.dout, b, h, i);
#pragma unroll
  for (int c = 0; c < DM; ++c) {
    qi[c] = c < d ? qp[c] : 0.f;
    gi[c] = c < d ? gp[c] : 0.f;
    dq[c] = 0.f;
  }
  const float li = a.lse[row_base + i], di = a.delta[row_base + i];
  int lo, hi;
  key_range(a.m, i, lo, hi);
  for (int j = lo; j < hi; ++j) {
    const float* kp = at<float>(a.k, b, h, j);
    const float* vp = at<float>(a.v, b, h, j);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < DM; ++c)
      if (c < d) {
        s = fmaf(qi[c], kp[c], s);
        dp = fmaf(gi[c], vp[c], dp);
      }
    const float p = expf(s * a.sm_scale - li);
    if (a.m.dropout) dp = dropout_keep(a.m, b, h, i, j) ? dp * a.m.keep_scale : 0.f;
    const float ds = p * (dp - di);
#pragma unroll
    for (int c = 0; c < DM; ++c)
      if (c < d) dq[c] = fmaf(ds, kp[c], dq[c]);
  }
  float* dqp = at<float>(a.dq, b, h, i);
#pragma unroll
  for (int c = 0; c < DM; ++c)
    if (c < d) dqp[c] = dq[c] * a.sm_scale;
}

template <int DM>
hipError_t launch_fwd_dm(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fwd_f32_kernel<DM>, dim3(a.B * a.H, (a.m.nq + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int DM>
hipError_t launch_bwd_dm(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dkdv_f32_kernel<DM>, dim3(a.B * a.H, (a.m.nk + 63) / 64), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_f32_kernel<DM>, dim3(a.B * a.H, (a.m.nq + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  if (a.d <= 32) return launch_fwd_dm<32>(a, s);
  if (a.d <= 64) return launch_fwd_dm<64>(a, s);
  return launch_fwd_dm<128>(a, s);
}

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s) {
  if (a.d <= 32) return launch_bwd_dm<32>(a, s);
  if (a.d <= 64) return launch_bwd_dm<64>(a, s);
  return launch_bwd_dm<128>(a, s);
}

}  // namespace fa
