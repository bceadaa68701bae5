// fa_prep.hip - HBM-bound helper kernels of the backward.
//
//  prep16_kernel,     D_i = sum_k dO_ik O_ik for every row, fp32 accumulate
//  prep_f32_kernel    ("FlashAttention backward", section "The gradients, and
//                     the one scalar that makes them local": a single
//                     streaming pass over O and dO ahead of the backward
//                     kernels), fused with zeroing the fp32 dQ accumulator of
//                     atomic mode.
//  dq_convert_kernel  dQ = round_to_dtype(sm_scale * dQ_acc) (bf16 or fp16).
//  mask_kernel        the dropout keep mask of one head (test aid).
//
// prep16_kernel (bf16/fp16, d = 64 or 128): d / 8 lanes per row, each lane
// one 16-byte chunk of O and of dO per row (fully coalesced rows), two rows
// per thread at d = 128 and four at d = 64 with every load issued before the
// first use; fp32 products, lane-shuffle reduction.  prep_f32_kernel covers fp32 and other d.  Rows
// are walked grid-stride so the grid can be sized to the machine.

#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kRowsPerBlock = 16;  // fp32 path: 256 threads, 16 lanes per row

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

// Packed row (b, h, n) of flat index `row`: its batch, head and sequence
// position (varlen: rows past sequence b's length hold no query, n < 0).
__device__ __forceinline__ void row_coords(const PrepArgs& a, int64_t row, int& b, int& h, int& n) {
  const int64_t HN = (int64_t)a.H * a.N;
  if (row < (int64_t)INT32_MAX && HN < (int64_t)INT32_MAX) {  // 32-bit division: a 64-bit one is a long software sequence
    const uint32_t r32 = (uint32_t)row, hn = (uint32_t)HN;
    b = (int)(r32 / hn);
    const uint32_t rem = r32 - (uint32_t)b * hn;
    h = (int)(rem / (uint32_t)a.N);
    n = (int)(rem - (uint32_t)h * (uint32_t)a.N);
  } else {
    b = (int)(row / HN);
    const int rem = (int)(row - b * HN);
    h = rem / a.N;
    n = rem - h * a.N;
  }
  if (a.cu_q) {
    const int q0 = a.cu_q[b];
    n = n < a.cu_q[b + 1] - q0 ? n + q0 : -1;
  }
}

// 16-bit rows: D / 8 lanes per row, each lane one 16-byte chunk of O and of
// dO per row, and R rows per thread whose loads are all issued before the
// first is used (more bytes in flight per thread: the pass is bound by HBM
// latency, not arithmetic).  The partial sums of a row's lanes are combined
// with lane shuffles.
template <typename T, typename T8, int D, int R, bool STREAM, bool CONTIG>
__global__ void __launch_bounds__(256) prep16_kernel(PrepArgs a) {
  constexpr int LPR = D / 8, SLOTS = 256 / LPR;  // lanes per row, rows per block pass
  const int sub = threadIdx.x % LPR, slot = threadIdx.x / LPR;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  for (int64_t base = (int64_t)blockIdx.x * SLOTS * R; base < rows; base += (int64_t)gridDim.x * SLOTS * R) {
    T8 ov[R], gv[R];
    int64_t rr[R];
    bool ok[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      rr[k] = base + slot + (int64_t)k * SLOTS;
      const T* op;
      const T* gp;
      if (CONTIG) {  // [B, H, N, d] without gaps: row r starts at r * d
        ok[k] = rr[k] < rows;
        op = (const T*)a.o.ptr + (ok[k] ? rr[k] : 0) * D;
        gp = (const T*)a.dout.ptr + (ok[k] ? rr[k] : 0) * D;
      } else {
        int b = 0, h = 0, n = -1;
        if (rr[k] < rows) row_coords(a, rr[k], b, h, n);
        ok[k] = n >= 0;
        // rows without a query read a valid row (their result is dropped):
        // an unconditional load does not make the thread wait for it here
        op = at<T>(a.o, b, h, ok[k] ? n : 0);
        gp = at<T>(a.dout, b, h, ok[k] ? n : 0);
      }
      if (STREAM) {  // read once: no reason to keep the lines in cache
        ov[k] = __builtin_nontemporal_load((const T8*)(op + 8 * sub));
        gv[k] = __builtin_nontemporal_load((const T8*)(gp + 8 * sub));
      } else {
        ov[k] = *(const T8*)(op + 8 * sub);
        gv[k] = *(const T8*)(gp + 8 * sub);
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (rr[k] >= rows) continue;
      float acc = 0.f;
      if (ok[k]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)ov[k][e], (float)gv[k][e], acc);
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
      if (ok[k] && sub == 0) a.delta[rr[k]] = acc;
      if (a.dq_acc) {  // atomic mode: this row of the fp32 dQ accumulator starts at zero
        f32x4* z = (f32x4*)(a.dq_acc + rr[k] * D) + 2 * sub;
        z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
}

// fp32 rows (any d): 16 lanes per row, grid-stride over rows.
__global__ void __launch_bounds__(256) prep_f32_kernel(PrepArgs a) {
  const int sub = threadIdx.x & 15;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4); row < rows;
       row += (int64_t)gridDim.x * kRowsPerBlock) {
    int b, h, n;
    row_coords(a, row, b, h, n);
    float acc = 0.f;
    if (n >= 0) {
      const float* op = at<float>(a.o, b, h, n);
      const float* gp = at<float>(a.dout, b, h, n);
      for (int c = sub; c < a.d; c += 16) acc = fmaf(op[c], gp[c], acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (n >= 0 && sub == 0) a.delta[row] = acc;
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

// Are a view's rows packed back to back in [B, H, N, d] order?
bool packed_rows(const TensorView& t, const PrepArgs& a) {
  return t.sn == a.d && t.sh == (int64_t)a.N * a.d && (a.B == 1 || t.sb == (int64_t)a.H * a.N * a.d);
}

}  // namespace

hipError_t launch_preprocess(const PrepArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const bool contig = !a.cu_q && packed_rows(a.o, a) && packed_rows(a.dout, a);
  if (a.dtype == 0 || (a.d != 64 && a.d != 128)) {
    hipLaunchKernelGGL(prep_f32_kernel, dim3(grid_for(rows, kRowsPerBlock)), dim3(256), 0, s, a);
  } else if (a.d == 128) {
    // 2 rows per thread (16 rows per block pass), measured best of 1, 2, 4, 8;
    // non-temporal loads (O and dO are read once here): 4.8 % faster alone,
    // the same whole step
    const dim3 grid(grid_for(rows, 16 * 2));
    if (a.dtype == 1)
      hipLaunchKernelGGL(contig ? (prep16_kernel<bf16, bf16x8, 128, 2, true, true>)
                                : (prep16_kernel<bf16, bf16x8, 128, 2, true, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(contig ? (prep16_kernel<f16, f16x8, 128, 2, true, true>)
                                : (prep16_kernel<f16, f16x8, 128, 2, true, false>), grid, dim3(256), 0, s, a);
  } else {
    // 4 rows per thread (32 rows per block pass), non-temporal loads
    const dim3 grid(grid_for(rows, 32 * 4));
    if (a.dtype == 1)
      hipLaunchKernelGGL(contig ? (prep16_kernel<bf16, bf16x8, 64, 4, true, true>)
                                : (prep16_kernel<bf16, bf16x8, 64, 4, true, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(contig ? (prep16_kernel<f16, f16x8, 64, 4, true, true>)
                                : (prep16_kernel<f16, f16x8, 64, 4, true, false>), grid, dim3(256), 0, s, a);
  }
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
