// fa_api.cpp - the C ABI of include/fa.h: argument validation, then launches.
//
// Every check runs before the first HIP call, so invalid arguments are
// reported without touching (or needing) a device.  After validation the
// only HIP calls are a device-count query and the kernel launches, each
// followed by a check of the launch status (a launch that is silently
// rejected would otherwise leave the outputs unwritten).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstddef>
#include <initializer_list>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr int64_t kMaxSeq = 1 << 21;  // keeps every launch within 65535 blocks per grid row

// Last HIP error seen by a call on this thread (diagnostics only).
thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// the 16-bit MFMA dtypes
bool is16(const fa_params* p) { return p->dtype == FA_DTYPE_BF16 || p->dtype == FA_DTYPE_F16; }

fa_status check_params(const fa_params* p) {
  if (!p) return FA_ERR_INVALID_VALUE;
  if (p->dtype != FA_DTYPE_F32 && p->dtype != FA_DTYPE_BF16 && p->dtype != FA_DTYPE_F16)
    return FA_ERR_NOT_SUPPORTED;
  if (p->batch < 1 || p->heads < 1 || p->seqlen < 1 || p->seqlen_k < 1 || p->head_dim < 1)
    return FA_ERR_INVALID_VALUE;
  if ((int64_t)p->batch * p->heads > INT32_MAX) return FA_ERR_NOT_SUPPORTED;
  if (p->seqlen > kMaxSeq || p->seqlen_k > kMaxSeq) return FA_ERR_NOT_SUPPORTED;
  // the kernels number their workgroups (one per head and 64 rows, plus up
  // to 3 blocks of padding per head) in an int
  const int64_t longest = p->seqlen > p->seqlen_k ? p->seqlen : p->seqlen_k;
  if ((int64_t)p->batch * p->heads * ((longest + 63) / 64 + 3) > INT32_MAX) return FA_ERR_NOT_SUPPORTED;
  // varlen: both offset arrays or neither
  if ((p->cu_seqlens_q == nullptr) != (p->cu_seqlens_k == nullptr)) return FA_ERR_INVALID_VALUE;
  if (p->cu_seqlens_q && (!aligned(p->cu_seqlens_q, 4) || !aligned(p->cu_seqlens_k, 4)))
    return FA_ERR_MISALIGNED;
  if (is16(p) && p->head_dim != 64 && p->head_dim != 128) return FA_ERR_NOT_SUPPORTED;
  if (p->dtype == FA_DTYPE_F32 && p->head_dim > 128) return FA_ERR_NOT_SUPPORTED;
  if (!std::isfinite(p->sm_scale)) return FA_ERR_INVALID_VALUE;
  if (p->window_left < -1 || p->window_right < -1) return FA_ERR_INVALID_VALUE;
  if (!(p->dropout_p >= 0.0 && p->dropout_p < 1.0)) return FA_ERR_INVALID_VALUE;
  if (p->dropout_p > 0.0) {
    if (std::ceil(p->dropout_p * 65536.0) > 65535.0) return FA_ERR_INVALID_VALUE;
    if (p->batch > 65536 || p->heads > 65536 || p->seqlen > 65536 || p->seqlen_k > 65536)
      return FA_ERR_NOT_SUPPORTED;
  }
  return FA_SUCCESS;
}

bool varlen(const fa_params* p) { return p->cu_seqlens_q != nullptr; }

// Atomic dQ mode (16-bit dtypes, deterministic == 0) accumulates dQ in an
// fp32 workspace; every other call has none.
bool uses_dq_acc(const fa_params* p) { return is16(p) && !p->deterministic; }

fa_status check_tensor(const fa_params* p, const fa_tensor& t) {
  if (!t.ptr) return FA_ERR_INVALID_VALUE;
  const int64_t sb = varlen(p) ? 0 : t.stride_b;  // varlen ignores the batch stride
  if (sb < 0 || t.stride_h < 0 || t.stride_n < 0) return FA_ERR_INVALID_VALUE;
  if (is16(p)) {
    if (!aligned(t.ptr, 16)) return FA_ERR_MISALIGNED;
    if ((sb % 8) || (t.stride_h % 8) || (t.stride_n % 8)) return FA_ERR_MISALIGNED;
    if (t.stride_n > INT32_MAX) return FA_ERR_NOT_SUPPORTED;  // row offsets are 32-bit products
  } else if (!aligned(t.ptr, 4)) {
    return FA_ERR_MISALIGNED;
  }
  return FA_SUCCESS;
}

fa_status check_vec(const float* v, uintptr_t align) {
  if (!v) return FA_ERR_INVALID_VALUE;
  if (!aligned(v, align)) return FA_ERR_MISALIGNED;
  return FA_SUCCESS;
}

// Detectable aliasing (equal base pointers): an output that is also an
// input, another output or one of the varlen offset arrays.  Null outputs
// (optional ones) are skipped.
bool aliased(const fa_params* p, std::initializer_list<const void*> outs,
             std::initializer_list<const void*> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    if (!*o) continue;
    if (*o == p->cu_seqlens_q || *o == p->cu_seqlens_k) return true;
    for (const void* i : ins)
      if (*o == i) return true;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (*o == *o2) return true;
  }
  return false;
}

#define FA_TRY(expr)                      \
  do {                                    \
    const fa_status st_ = (expr);         \
    if (st_ != FA_SUCCESS) return st_;    \
  } while (0)

// varlen views carry no batch stride: sequence b's rows are located by the
// offset arrays instead
fa::TensorView view(const fa_params* p, const fa_tensor& t) {
  return fa::TensorView{t.ptr, varlen(p) ? 0 : t.stride_b, t.stride_h, t.stride_n};
}

fa::MaskArgs mask_args(const fa_params* p) {
  fa::MaskArgs m{};
  m.nq = p->seqlen;
  m.nk = p->seqlen_k;
  m.causal = p->causal ? 1 : 0;
  // visible iff i' - window_left <= j <= i' + window_right (j <= i' if
  // causal), with i' = i + nk - nq; the kernels add that shift per sequence.
  // 2^30 stands for unbounded (|nk - nq| < 2^21 keeps every sum in range).
  m.lo_off = p->window_left >= 0 ? p->window_left : (1 << 30);
  m.hi_off = p->window_right >= 0 ? p->window_right : (1 << 30);
  if (p->causal && m.hi_off > 0) m.hi_off = 0;
  m.cu_q = p->cu_seqlens_q;
  m.cu_k = p->cu_seqlens_k;
  m.dropout = p->dropout_p > 0.0 ? 1 : 0;
  m.keep_threshold = (uint32_t)std::ceil(p->dropout_p * 65536.0);  // of a 16-bit draw
  m.keep_scale = (float)(1.0 / (1.0 - p->dropout_p));
  m.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFull);
  m.seed_hi = (uint32_t)(p->seed >> 32);
  m.off_lo = (uint32_t)(p->offset & 0xFFFFFFFFull);
  m.off_hi = (uint32_t)(p->offset >> 32);
  return m;
}

// A usable device must exist before anything is launched.
fa_status device_ready() {
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n < 1) {
    g_last_hip_error = e != hipSuccess ? (int)e : (int)hipErrorNoDevice;
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return FA_ERR_HIP;
  }
  return FA_SUCCESS;
}

fa_status launched(hipError_t e) {
  if (e == hipSuccess) return FA_SUCCESS;
  g_last_hip_error = (int)e;
  if (e == hipErrorLaunchFailure || e == hipErrorInvalidConfiguration || e == hipErrorInvalidValue ||
      e == hipErrorLaunchOutOfResources || e == hipErrorInvalidDeviceFunction)
    return FA_ERR_LAUNCH_FAILED;
  return FA_ERR_HIP;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

int fa_last_hip_error(void) { return g_last_hip_error; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_SUCCESS: return "success";
    case FA_ERR_INVALID_VALUE: return "invalid argument value";
    case FA_ERR_NOT_SUPPORTED: return "configuration not supported";
    case FA_ERR_MISALIGNED: return "pointer or stride misaligned";
    case FA_ERR_LAUNCH_FAILED: return "kernel launch failed";
    case FA_ERR_HIP: return "HIP runtime error (no usable device?)";
    case FA_ERR_TOO_LARGE: return "dQ workspace larger than FA_STATIC_WORKSPACE_BYTES";
  }
  return "unknown status";
}

fa_status fa_fwd(const fa_params* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                 void* stream) {
  FA_TRY(check_params(p));
  FA_TRY(check_tensor(p, q));
  FA_TRY(check_tensor(p, k));
  FA_TRY(check_tensor(p, v));
  FA_TRY(check_tensor(p, o));
  FA_TRY(check_vec(lse, 4));
  if (aliased(p, {o.ptr, lse}, {q.ptr, k.ptr, v.ptr})) return FA_ERR_INVALID_VALUE;
  FA_TRY(device_ready());
  fa::FwdArgs a{};
  a.q = view(p, q);
  a.k = view(p, k);
  a.v = view(p, v);
  a.o = view(p, o);
  a.lse = lse;
  a.B = p->batch;
  a.H = p->heads;
  a.d = p->head_dim;
  a.ln = p->seqlen;
  a.sm_scale = p->sm_scale;
  a.scale_log2 = p->sm_scale * kLog2e;
  a.m = mask_args(p);
  hipStream_t s = (hipStream_t)stream;
  if (p->dtype == FA_DTYPE_BF16) return launched(fa::launch_fwd16(a, s));
  if (p->dtype == FA_DTYPE_F16) return launched(fa::fp16::launch_fwd16(a, s));
  return launched(fa::launch_fwd_f32(a, s));
}

size_t fa_bwd_workspace_bytes(const fa_params* p) {
  if (check_params(p) != FA_SUCCESS) return 0;
  if (!uses_dq_acc(p)) return 0;
  return (size_t)4 * (size_t)p->batch * (size_t)p->heads * (size_t)p->seqlen * (size_t)p->head_dim;
}

fa_status fa_bwd_preprocess(const fa_params* p, fa_tensor o, fa_tensor dout, float* delta, float* dq_acc,
                            void* stream) {
  FA_TRY(check_params(p));
  FA_TRY(check_tensor(p, o));
  FA_TRY(check_tensor(p, dout));
  FA_TRY(check_vec(delta, 4));
  // the accumulator exists only in atomic mode; any other pointer is ignored
  if (!uses_dq_acc(p)) dq_acc = nullptr;
  if (dq_acc) FA_TRY(check_vec(dq_acc, 16));
  if (aliased(p, {delta, dq_acc}, {o.ptr, dout.ptr})) return FA_ERR_INVALID_VALUE;
  FA_TRY(device_ready());
  fa::PrepArgs a{};
  a.o = view(p, o);
  a.dout = view(p, dout);
  a.delta = delta;
  a.dq_acc = dq_acc;
  a.cu_q = p->cu_seqlens_q;
  a.B = p->batch;
  a.H = p->heads;
  a.N = p->seqlen;
  a.d = p->head_dim;
  a.dtype = p->dtype;
  a.sm_scale = p->sm_scale;
  return launched(fa::launch_preprocess(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Every check of fa_bwd except the workspace's.
fa_status check_bwd(const fa_params* p, const fa_tensor& q, const fa_tensor& k, const fa_tensor& v,
                    const fa_tensor& dout, const float* lse, const float* delta, const fa_tensor& dq,
                    const fa_tensor& dk, const fa_tensor& dv) {
  FA_TRY(check_params(p));
  FA_TRY(check_tensor(p, q));
  FA_TRY(check_tensor(p, k));
  FA_TRY(check_tensor(p, v));
  FA_TRY(check_tensor(p, dout));
  FA_TRY(check_tensor(p, dq));
  FA_TRY(check_tensor(p, dk));
  FA_TRY(check_tensor(p, dv));
  FA_TRY(check_vec(lse, 4));
  FA_TRY(check_vec(delta, 4));
  if (aliased(p, {dq.ptr, dk.ptr, dv.ptr}, {q.ptr, k.ptr, v.ptr, dout.ptr, lse, delta}))
    return FA_ERR_INVALID_VALUE;
  return FA_SUCCESS;
}

// The launches of fa_bwd, after validation; dq_acc is the (zeroed) fp32
// workspace in atomic mode, else ignored.
fa_status run_bwd(const fa_params* p, const fa_tensor& q, const fa_tensor& k, const fa_tensor& v,
                  const fa_tensor& dout, const float* lse, const float* delta, const fa_tensor& dq,
                  const fa_tensor& dk, const fa_tensor& dv, float* dq_acc, hipStream_t s) {
  const bool atomic = uses_dq_acc(p);
  fa::BwdArgs a{};
  a.q = view(p, q);
  a.k = view(p, k);
  a.v = view(p, v);
  a.dout = view(p, dout);
  a.dq = view(p, dq);
  a.dk = view(p, dk);
  a.dv = view(p, dv);
  a.lse = lse;
  a.delta = delta;
  a.dq_acc = atomic ? dq_acc : nullptr;
  a.B = p->batch;
  a.H = p->heads;
  a.d = p->head_dim;
  a.ln = p->seqlen;
  a.sm_scale = p->sm_scale;
  a.scale_log2 = p->sm_scale * kLog2e;
  a.m = mask_args(p);
  if (p->dtype == FA_DTYPE_F32) return launched(fa::launch_bwd_f32(a, s));
  FA_TRY(launched(p->dtype == FA_DTYPE_F16 ? fa::fp16::launch_bwd16(a, !atomic, s)
                                             : fa::launch_bwd16(a, !atomic, s)));
  if (atomic) {
    fa::PrepArgs c{};
    c.dq = view(p, dq);
    c.dq_acc = dq_acc;
    c.cu_q = p->cu_seqlens_q;
    c.B = p->batch;
    c.H = p->heads;
    c.N = p->seqlen;
    c.d = p->head_dim;
    c.dtype = p->dtype;
    // under dropout the KV-outer kernel accumulates dS (1 - p): 1 / (1 - p) here
    c.sm_scale = p->sm_scale * a.m.keep_scale;
    FA_TRY(launched(fa::launch_dq_convert(c, s)));
  }
  return FA_SUCCESS;
}

}  // namespace

extern "C" {

fa_status fa_bwd(const fa_params* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor dout, const float* lse,
                 const float* delta, fa_tensor dq, fa_tensor dk, fa_tensor dv, float* dq_acc, void* stream) {
  FA_TRY(check_bwd(p, q, k, v, dout, lse, delta, dq, dk, dv));
  const bool atomic = uses_dq_acc(p);
  if (atomic) {
    FA_TRY(check_vec(dq_acc, 16));
    if (aliased(p, {dq_acc}, {q.ptr, k.ptr, v.ptr, dout.ptr, lse, delta, dq.ptr, dk.ptr, dv.ptr}))
      return FA_ERR_INVALID_VALUE;
  }
  FA_TRY(device_ready());
  return run_bwd(p, q, k, v, dout, lse, delta, dq, dk, dv, dq_acc, (hipStream_t)stream);
}

fa_status fa_bwd_noalloc(const fa_params* p, fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor dout,
                         const float* lse, const float* delta, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                         void* stream) {
  FA_TRY(check_bwd(p, q, k, v, dout, lse, delta, dq, dk, dv));
  const size_t ws = fa_bwd_workspace_bytes(p);
  if (ws > FA_STATIC_WORKSPACE_BYTES) return FA_ERR_TOO_LARGE;
  FA_TRY(device_ready());
  hipStream_t s = (hipStream_t)stream;
  float* scratch = nullptr;
  if (ws) {
    // this device's copy of the static array, then clear the part in use
    const hipError_t e = fa::static_workspace(&scratch);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return FA_ERR_HIP;
    }
    FA_TRY(launched(fa::launch_zero(scratch, ws, s)));
  }
  return run_bwd(p, q, k, v, dout, lse, delta, dq, dk, dv, scratch, s);
}

fa_status fa_debug_dropout_mask(const fa_params* p, int32_t b, int32_t h, uint8_t* mask, void* stream) {
  FA_TRY(check_params(p));
  if (!mask) return FA_ERR_INVALID_VALUE;
  if (b < 0 || b >= p->batch || h < 0 || h >= p->heads) return FA_ERR_INVALID_VALUE;
  if (p->seqlen > 65536 || p->seqlen_k > 65536 || p->batch > 65536 || p->heads > 65536)
    return FA_ERR_NOT_SUPPORTED;
  FA_TRY(device_ready());
  return launched(fa::launch_dropout_mask(mask_args(p), b, h, mask, (hipStream_t)stream));
}

}  // extern "C"
