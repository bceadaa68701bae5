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

// Visible key range [lo, hi) of query row i.
__device__ __forceinline__ void key_range(const MaskArgs& m, int i, int& lo, int& hi) {
  lo = 0;
  hi = m.n;
  if (m.causal) hi = min(hi, i + 1);
  if (m.wl >= 0) lo = max(lo, i - m.wl);
  if (m.wr >= 0) hi = min(hi, i + m.wr + 1);
}

// Query range [lo, hi) that sees key row j.
__device__ __forceinline__ void query_range(const MaskArgs& m, int j, int& lo, int& hi) {
  lo = 0;
  hi = m.n;
  if (m.causal) lo = max(lo, j);
  if (m.wr >= 0) lo = max(lo, j - m.wr);
  if (m.wl >= 0) hi = min(hi, j + m.wl + 1);
}

template <int DM>
__global__ void __launch_bounds__(64) fwd_f32_kernel(FwdArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H;
  const int i = blockIdx.y * 64 + threadIdx.x;
  const int N = a.m.n, d = a.d;
  if (i >= N) return;
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
  float* op = at<float>(a.o, b, h, i);
  const float inv = 1.f / l_run;
#pragma unroll
  for (int c = 0; c < DM; ++c)
    if (c < d) op[c] = o[c] * inv;
  a.lse[(int64_t)bh * N + i] = m_run + logf(l_run);
}

template <int DM>
__global__ void __launch_bounds__(64) dkdv_f32_kernel(BwdArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H;
  const int j = blockIdx.y * 64 + threadIdx.x;
  const int N = a.m.n, d = a.d;
  if (j >= N) return;
  const int64_t row_base = (int64_t)bh * N;
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
  const int i = blockIdx.y * 64 + threadIdx.x;
  const int N = a.m.n, d = a.d;
  if (i >= N) return;
  const int64_t row_base = (int64_t)bh * N;
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
  hipLaunchKernelGGL(fwd_f32_kernel<DM>, dim3(a.B * a.H, (a.m.n + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int DM>
hipError_t launch_bwd_dm(const BwdArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H, (a.m.n + 63) / 64);
  hipLaunchKernelGGL(dkdv_f32_kernel<DM>, grid, dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_f32_kernel<DM>, grid, dim3(64), 0, s, a);
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
