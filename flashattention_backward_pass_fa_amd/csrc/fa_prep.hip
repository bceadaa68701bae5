// fa_prep.hip - HBM-bound helper kernels of the backward.
//
//  prep_kernel        D_i = sum_k dO_ik O_ik for every row, fp32 accumulate
//                     ("FlashAttention backward", section "The gradients, and
//                     the one scalar that makes them local": a single
//                     streaming pass over O and dO ahead of the backward
//                     kernels), fused with zeroing the fp32 dQ accumulator of
//                     atomic mode.
//  dq_convert_kernel  dQ = round_to_dtype(sm_scale * dQ_acc) (bf16 or fp16).
//  mask_kernel        the dropout keep mask of one head (test aid).
//
// prep_kernel: 16 lanes per row, each lane loads 16 contiguous bytes of O
// and dO per step (fully coalesced rows), multiplies in fp32, and the 16
// partial sums are combined with lane shuffles.  Rows are walked
// grid-stride so the grid can be sized to the machine.

#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kRowsPerBlock = 16;  // 256 threads, 16 lanes per row

// this lane's share of sum_k dO_k O_k over a 16-bit row (8 elements per step)
template <typename T, typename T8>
__device__ __forceinline__ float row_dot16(const TensorView& o, const TensorView& g, int b, int h, int n,
                                           int d, int sub) {
  const T* op = at<T>(o, b, h, n);
  const T* gp = at<T>(g, b, h, n);
  float acc = 0.f;
  for (int c0 = sub * 8; c0 < d; c0 += 128) {
    const T8 ov = *(const T8*)(op + c0);
    const T8 gv = *(const T8*)(gp + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)ov[e], (float)gv[e], acc);
  }
  return acc;
}

template <typename T, typename T8>
__device__ __forceinline__ void store_scaled8(T* dst, f32x4 x0, f32x4 x1, float scale) {
  T8 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[e] = (T)(x0[e] * scale);
    y[4 + e] = (T)(x1[e] * scale);
  }
  *(T8*)dst = y;
}

// zero one row of the fp32 dQ accumulator (atomic mode), 16 lanes per row
__device__ __forceinline__ void zero_acc_row(const PrepArgs& a, int64_t row, int sub) {
  if (!a.dq_acc) return;
  float* zrow = a.dq_acc + row * a.d;
  if ((a.d & 3) == 0) {
    for (int c4 = sub; c4 * 4 < a.d; c4 += 16) ((f32x4*)zrow)[c4] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int c = sub; c < a.d; c += 16) zrow[c] = 0.f;
  }
}

__global__ void __launch_bounds__(256) prep_kernel(PrepArgs a) {
  const int sub = threadIdx.x & 15;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int64_t HN = (int64_t)a.H * a.N;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4); row < rows;
       row += (int64_t)gridDim.x * kRowsPerBlock) {
    const int b = (int)(row / HN);
    const int rem = (int)(row - b * HN);
    const int h = rem / a.N;
    int n = rem - h * a.N;
    if (a.cu_q) {  // varlen: rows past sequence b's length hold no query
      const int q0 = a.cu_q[b];
      if (n >= a.cu_q[b + 1] - q0) {
        zero_acc_row(a, row, sub);
        continue;
      }
      n += q0;
    }
    float acc = 0.f;
    if (a.dtype == 1) {
      acc = row_dot16<bf16, bf16x8>(a.o, a.dout, b, h, n, a.d, sub);
    } else if (a.dtype == 2) {
      acc = row_dot16<f16, f16x8>(a.o, a.dout, b, h, n, a.d, sub);
    } else {
      const float* op = at<float>(a.o, b, h, n);
      const float* gp = at<float>(a.dout, b, h, n);
      for (int c = sub; c < a.d; c += 16) acc = fmaf(op[c], gp[c], acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (sub == 0) a.delta[row] = acc;
    zero_acc_row(a, row, sub);
  }
}

__global__ void __launch_bounds__(256) dq_convert_kernel(PrepArgs a) {
  // one thread per 8 consecutive elements of a row
  const int per_row = a.d / 8;
  const int64_t total = (int64_t)a.B * a.H * a.N * per_row;
  const int64_t HN = (int64_t)a.H * a.N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / per_row;
    const int c0 = (int)(t - row * per_row) * 8;
    const int b = (int)(row / HN);
    const int rem = (int)(row - b * HN);
    const int h = rem / a.N;
    int n = rem - h * a.N;
    if (a.cu_q) {  // varlen: rows past sequence b's length hold no query
      const int q0 = a.cu_q[b];
      if (n >= a.cu_q[b + 1] - q0) continue;
      n += q0;
    }
    const f32x4* src = (const f32x4*)(a.dq_acc + row * a.d + c0);
    const f32x4 x0 = src[0], x1 = src[1];
    if (a.dtype == 2)
      store_scaled8<f16, f16x8>(at<f16>(a.dq, b, h, n) + c0, x0, x1, a.sm_scale);
    else
      store_scaled8<bf16, bf16x8>(at<bf16>(a.dq, b, h, n) + c0, x0, x1, a.sm_scale);
  }
}

__global__ void __launch_bounds__(256) mask_kernel(MaskArgs m, int b, int h, uint8_t* out) {
  const int i = blockIdx.x;
  const int j = blockIdx.y * 256 + threadIdx.x;
  if (j < m.nk) out[(int64_t)i * m.nk + j] = dropout_keep(m, b, h, i, j) ? 1 : 0;
}

int grid_for(int64_t work_items, int per_block) {
  int64_t blocks = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 32;  // enough resident blocks to cover 256 CUs many times
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

hipError_t launch_preprocess(const PrepArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  hipLaunchKernelGGL(prep_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dq_convert(const PrepArgs& a, hipStream_t s) {
  const int64_t items = (int64_t)a.B * a.H * a.N * (a.d / 8);
  hipLaunchKernelGGL(dq_convert_kernel, dim3(grid_for(items, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dropout_mask(const MaskArgs& m, int b, int h, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(mask_kernel, dim3(m.nq, (m.nk + 255) / 256), dim3(256), 0, s, m, b, h, out);
  return hipGetLastError();
}

}  // namespace fa
