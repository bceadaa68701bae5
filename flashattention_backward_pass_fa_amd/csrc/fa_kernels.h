// fa_kernels.h - argument blocks and host-side launchers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {

// Arguments of the forward kernels.
struct FwdArgs {
  TensorView q, k, v, o;
  float* lse;          // [B, H, ln] fp32
  int B, H, d;
  int ln;              // rows per head of L (the longest query sequence)
  float sm_scale;
  float scale_log2;    // sm_scale * log2(e)
  MaskArgs m;
};

// Arguments of the backward kernels.
struct BwdArgs {
  TensorView q, k, v, dout, dq, dk, dv;
  const float* lse;    // [B, H, ln] fp32, natural log
  const float* delta;  // [B, H, ln] fp32
  float* dq_acc;       // [B, H, ln, d] fp32 (atomic mode)
  int B, H, d;
  int ln;              // rows per head of L, D and dq_acc (the longest query sequence)
  float sm_scale;
  float scale_log2;
  MaskArgs m;
};

// Arguments of the pre-pass (D) and the dQ conversion.
struct PrepArgs {
  TensorView o, dout, dq;
  float* delta;        // [B, H, N] fp32
  float* dq_acc;       // [B, H, N, d] fp32
  const int* cu_q;     // varlen: sequence b has packed rows [cu_q[b], cu_q[b+1]); else null
  int B, H, N, d;      // N: rows per head of delta and dq_acc (the longest query sequence)
  int dtype;           // element type of o/dout/dq: 0 fp32, 1 bf16, 2 fp16 (fa_dtype)
  float sm_scale;
};

// Launchers: return hipSuccess or the launch error.  No validation here;
// the C-ABI layer validates every argument first.
hipError_t launch_fwd16(const FwdArgs& a, hipStream_t s);  // bf16 (fp16: in namespace fp16)
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd16(const BwdArgs& a, bool deterministic, hipStream_t s);
hipError_t launch_kv128(const BwdArgs& a, hipStream_t s);  // KV-outer, d = 128, deterministic
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s);
namespace fp16 {
hipError_t launch_fwd16(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd16(const BwdArgs& a, bool deterministic, hipStream_t s);
hipError_t launch_kv128(const BwdArgs& a, hipStream_t s);
}  // namespace fp16
hipError_t launch_preprocess(const PrepArgs& a, hipStream_t s);
hipError_t launch_dq_convert(const PrepArgs& a, hipStream_t s);
hipError_t launch_dropout_mask(const MaskArgs& m, int b, int h, uint8_t* out, hipStream_t s);

// The static fp32 workspace of fa_bwd_noalloc (fa_noalloc.hip): its device
// address on the current device (looked up once per device), and a kernel
// that zeroes the first `bytes` (a multiple of 16) of a buffer.
hipError_t static_workspace(float** out);
hipError_t launch_zero(float* p, size_t bytes, hipStream_t s);

}  // namespace fa
