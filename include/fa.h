/*
 * fa.h - FlashAttention forward/backward on AMD MI355X (gfx950), C ABI.
 *
 * The backward computes dQ, dK, dV of softmax attention from Q, K, V, the
 * forward output O, the upstream gradient dO and the per-row log-sum-exp L,
 * with O(N d) extra memory: each S/P tile is recomputed on chip as
 * P_ij = exp(S_ij - L_i), with the per-row scalar D_i = sum_k dO_ik O_ik, and
 * dS = P * (dP - D).  The N x N matrices are never written to memory.
 *
 *   "Lecture 7 - Backward Pass and Validation": sections "The math"
 *   (gradients), "The recomputation trick" (recompute P from the saved LSE),
 *   "Determinism", "Dropout", "Mask behaviour".
 *   "FlashAttention backward" (GPU kernels lesson 29): sections "What the
 *   forward left behind" (O and L_i = m_i + log l_i), "The gradients, and the
 *   one scalar that makes them local" (D), "The loop structure" (KV-outer
 *   loop; dQ by atomics or by a separate Q-outer kernel).
 *   Lecture 7's section on the FA test suite lists variable-length batches
 *   among the features a harness covers; the pages define no convention for
 *   them, so the one below is this library's (see fa_params).
 *
 * Conventions shared by every entry point
 *   - Tensors Q, K, V, O, dO, dQ, dK, dV are described by fa_tensor: a device
 *     pointer and element strides for the batch, head and sequence axes; the
 *     head-dim axis has stride 1.  [B,H,N,d] contiguous and [B,N,H,d] are
 *     both expressible.  Q, O, dO, dQ have N = seqlen rows per head and
 *     K, V, dK, dV have N = seqlen_k (or, in varlen mode, the packed rows
 *     of fa_params).  bf16 and fp16 tensors need a 16-byte aligned
 *     pointer and strides that are multiples of 8 elements, and fit each
 *     row stride in 32 bits of bytes; fp32 tensors need 4-byte alignment.
 *   - L (lse), D (delta) are fp32, [B,H,seqlen] contiguous.  L is the natural
 *     log of sum_j exp(S_ij) over the visible keys of row i, with
 *     S = sm_scale * Q K^T; a row that sees no key has L = -inf, O = 0 and
 *     dQ = 0.
 *   - Ownership: the caller allocates every buffer (device memory) and keeps
 *     it alive until the work on `stream` completes.  The library allocates
 *     no device memory and keeps no caller pointer after a call returns;
 *     calls are re-entrant.  Its only global state is fa_bwd_noalloc's static
 *     workspace (see there) and the per-device address of it.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and the call returns after launch.  Kernels run on the
 *     calling thread's current HIP device: the buffers and `stream` must
 *     belong to it.  FA_SUCCESS means
 *     the arguments were valid and every launch was accepted; faults during
 *     execution surface at the caller's next synchronisation.
 *   - Errors: every argument is validated before any HIP call, so a bad
 *     argument returns FA_ERR_INVALID_VALUE / FA_ERR_NOT_SUPPORTED /
 *     FA_ERR_MISALIGNED without touching the device.  A failed launch
 *     returns FA_ERR_LAUNCH_FAILED, any other HIP error FA_ERR_HIP.  The
 *     library never aborts and never prints.
 *   - Outputs must not alias inputs, each other or the varlen offset arrays;
 *     aliasing that shows as equal base pointers returns
 *     FA_ERR_INVALID_VALUE.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 3

/* Size of the static device workspace of fa_bwd_noalloc (per GPU). */
#define FA_STATIC_WORKSPACE_BYTES (128u * 1024u * 1024u)

typedef enum fa_status {
  FA_SUCCESS = 0,
  FA_ERR_INVALID_VALUE = 1,  /* null pointer, bad size, stride, window, p */
  FA_ERR_NOT_SUPPORTED = 2,  /* valid but not implemented (dtype, head dim) */
  FA_ERR_MISALIGNED = 3,     /* pointer or stride alignment */
  FA_ERR_LAUNCH_FAILED = 4,  /* a kernel launch was rejected */
  FA_ERR_HIP = 5,            /* another HIP runtime error (e.g. no device) */
  FA_ERR_TOO_LARGE = 6       /* fa_bwd_noalloc: the problem's workspace exceeds
                                FA_STATIC_WORKSPACE_BYTES */
} fa_status;

typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,   /* fp32 inputs/outputs, fp32 arithmetic */
  FA_DTYPE_BF16 = 1,  /* bf16 inputs/outputs, bf16 MFMA with fp32 accumulation */
  FA_DTYPE_F16 = 2    /* fp16 inputs/outputs, fp16 MFMA with fp32 accumulation */
} fa_dtype;

/* One tensor of logical shape [B, H, N, d]; element (b, h, n, c) lives at
 * ptr + b*stride_b + h*stride_h + n*stride_n + c (in elements). */
typedef struct fa_tensor {
  void* ptr;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_n;
} fa_tensor;

/* Flags and sizes of one attention call.
 *   dtype         FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16
 *   batch, heads  B, H >= 1
 *   seqlen        Nq, queries per sequence, 1 <= Nq <= 2^21
 *   seqlen_k      Nk, keys per sequence, 1 <= Nk <= 2^21;
 *                 B * H * (ceil(max(Nq, Nk) / 64) + 3) must stay below 2^31
 *   head_dim      d: bf16 and fp16 support 64 and 128; fp32 supports 1..128
 *   sm_scale      S = sm_scale * Q K^T (the pages use 1/sqrt(d)); any finite
 *                 value, 0 included
 *   Masks align the last query with the last key: query i stands at key
 *   position i' = i + Nk - Nq (i' = i when Nq = Nk).
 *   causal        non-zero: key j is hidden from query i when j > i'
 *   window_left   -1 = unbounded, else keys j >= i' - window_left only
 *   window_right  -1 = unbounded, else keys j <= i' + window_right only
 *                 (with Nq = Nk and windows >= 0 key i is always visible;
 *                 with Nq > Nk, or a window that misses [0, Nk), a row can
 *                 see no key)
 *   dropout_p     probability of dropping an attention weight, in
 *                 [0, 1 - 2^-16]; kept weights are scaled by 1/(1 - p).
 *                 Requires B, H, Nq, Nk <= 65536 when p > 0.
 *   seed, offset  Philox4x32-10 stream of the dropout mask: key = seed,
 *                 one block per eight keys j8 = j - j % 8, counter =
 *                 (offset, (i << 16) | j8, (b << 16) | h); weight
 *                 (b, h, i, j) draws the 16-bit half j % 2 (low first) of
 *                 word (j % 8) / 2 and is kept iff that draw >=
 *                 ceil(p * 2^16) (kept with probability within 2^-16 of
 *                 1 - p); i and j count from the start of the sequence.
 *   deterministic non-zero: dQ by a separate Q-outer kernel, bit-identical
 *                 run to run; zero: for bf16/fp16, dQ by fp32 atomics into
 *                 a workspace (fp32 computes dQ without atomics either way).
 *   cu_seqlens_q, cu_seqlens_k
 *                 NULL (both): every sequence has Nq queries and Nk keys at
 *                 tensor rows 0.. of its batch index.  Non-NULL (both):
 *                 varlen mode, device arrays of B + 1 int32 each; sequence b
 *                 has queries at packed rows [cu_seqlens_q[b],
 *                 cu_seqlens_q[b+1]) and keys at [cu_seqlens_k[b],
 *                 cu_seqlens_k[b+1]) of the tensors (row r of head h at
 *                 ptr + h*stride_h + r*stride_n; stride_b is ignored), and
 *                 seqlen / seqlen_k are the longest lengths.  Lengths are
 *                 clamped to [0, seqlen] / [0, seqlen_k] and each sequence
 *                 aligns its own last query and key.  L, D and the dQ
 *                 workspace keep the [B,H,seqlen] layout: entries past a
 *                 sequence's length are not written.  The caller keeps the
 *                 arrays (and every packed row they name) valid until the
 *                 work completes; they cannot be checked without a copy to
 *                 the host.
 */
typedef struct fa_params {
  int32_t dtype;
  int32_t batch;
  int32_t heads;
  int32_t seqlen;
  int32_t seqlen_k;
  int32_t head_dim;
  float sm_scale;
  int32_t causal;
  int32_t window_left;
  int32_t window_right;
  int32_t deterministic;
  double dropout_p;
  uint64_t seed;
  uint64_t offset;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
} fa_params;

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

/* The hipError_t code behind the last FA_ERR_HIP / FA_ERR_LAUNCH_FAILED
 * returned on the calling thread (0 if none); diagnostics only. */
int fa_last_hip_error(void);

/* Static, never-NULL description of a status code. */
const char* fa_status_string(fa_status status);

/* Forward: O = (P * Z / (1 - p)) V with P = softmax of the masked scores, and
 * L_i = m_i + log l_i ("FlashAttention backward", "What the forward left
 * behind").  o: output in the input dtype; lse: fp32 [B,H,N] output. */
fa_status fa_fwd(const fa_params* params, fa_tensor q, fa_tensor k, fa_tensor v,
                 fa_tensor o, float* lse, void* stream);

/* Backward pre-pass: D_i = sum_k dO_ik * O_ik, one fp32 scalar per row,
 * accumulated in fp32 ("FlashAttention backward", "The gradients, and the
 * one scalar that makes them local").  delta: fp32 [B,H,N] output.
 * dq_acc: the fp32 workspace of fa_bwd when fa_bwd_workspace_bytes(params)
 * is not 0 (bf16/fp16 with deterministic == 0), which this call then zeroes and
 * which that fa_bwd requires zeroed; NULL there skips the zeroing.  For
 * every other params it is ignored and never written (may be NULL). */
fa_status fa_bwd_preprocess(const fa_params* params, fa_tensor o, fa_tensor dout,
                            float* delta, float* dq_acc, void* stream);

/* Bytes of fp32 workspace fa_bwd needs: 4*B*H*seqlen*d for bf16/fp16 with
 * deterministic == 0 (the dQ accumulator, [B,H,seqlen,d] contiguous), else
 * 0 (also 0 when params are invalid). */
size_t fa_bwd_workspace_bytes(const fa_params* params);

/* Backward: dQ, dK, dV in the input dtype ("Lecture 7", "The math";
 * "FlashAttention backward", "The loop structure").  lse: L from fa_fwd;
 * delta: D from fa_bwd_preprocess.  dq_acc: required when
 * fa_bwd_workspace_bytes(params) is not 0, zeroed by fa_bwd_preprocess
 * beforehand; ignored (may be NULL) otherwise.  dK and dV are bit-reproducible run to run in both modes. */
fa_status fa_bwd(const fa_params* params, fa_tensor q, fa_tensor k, fa_tensor v,
                 fa_tensor dout, const float* lse, const float* delta,
                 fa_tensor dq, fa_tensor dk, fa_tensor dv, float* dq_acc,
                 void* stream);

/* fa_bwd without the caller's workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments as fa_bwd except
 * dq_acc, the same results.  Where fa_bwd needs its fp32 dQ workspace
 * (fa_bwd_workspace_bytes(params) != 0: bf16/fp16 with deterministic == 0),
 * this call uses a static device array of FA_STATIC_WORKSPACE_BYTES that the
 * library holds on every GPU it runs on until the process ends, and clears
 * the part it uses with a kernel on `stream` first; a larger workspace
 * returns FA_ERR_TOO_LARGE before any HIP call.  Every other params needs no
 * workspace and runs exactly as fa_bwd.  D comes from fa_bwd_preprocess as
 * for fa_bwd (its dq_acc may be NULL).  The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine; its first call on a
 * device looks up that device's array once.  All calls on one GPU share that
 * GPU's array, so calls that overlap on one GPU (on different streams, or
 * from several threads without ordering) race and give wrong dQ; order them
 * on one stream. */
fa_status fa_bwd_noalloc(const fa_params* params, fa_tensor q, fa_tensor k, fa_tensor v,
                         fa_tensor dout, const float* lse, const float* delta,
                         fa_tensor dq, fa_tensor dk, fa_tensor dv, void* stream);

/* Test aid, O(Nq Nk) by design: writes the Nq x Nk keep mask Z (1 = kept,
 * 0 = dropped; row i = query, column j = key) of head (b, h) to device
 * memory `mask` (uint8, row-major), using the same device function as the
 * kernels.  Masked-out (invisible) pairs are still written with their
 * Philox value; varlen offsets play no part (b is the sequence index). */
fa_status fa_debug_dropout_mask(const fa_params* params, int32_t b, int32_t h,
                                uint8_t* mask, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
