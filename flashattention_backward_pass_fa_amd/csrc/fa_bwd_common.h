// fa_bwd_common.h - device helpers shared by the backward kernel sources
// (fa_bwd16.hip, fa_kv128.hip): 16-byte LDS/global moves, the block-level
// mask tests, and the specialisation of a call to one sequence.
#pragma once

#include "fa_kernels.h"

namespace fa {
FA_ELEM_NS_BEGIN
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt operand (gfx9 encoding) that waits for every outstanding vector
// memory load and nothing else: vmcnt 0, expcnt 7, lgkmcnt 15.
constexpr int kVmcntZero = 0x0F70;




__device__ __forceinline__ e16x8 load8(const e16* p) { return *(const e16x8*)p; }
__device__ __forceinline__ void store8(e16* p, e16x8 v) { *(e16x8*)p = v; }

__device__ __forceinline__ e16x8 zero8() {
  e16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (e16)0.0f;
  return z;
}

// The KV-outer kernels read rows past a sequence's end as copies of its
// last row (a clamped index) rather than under a condition: a load under a
// condition compiles to a branch that waits for it, which turned their
// prologues into one memory round trip per load.  The copies are finite and
// every use of them is masked or lands in rows that are never stored.  (The
// Q-outer kernel keeps zero rows: its clamped form measured slower.)

// Is every (query, key) of rows [q0, q0+rows) x keys [k0, k0+cols) visible?
__device__ __forceinline__ bool block_full(const MaskArgs& m, int q0, int rows, int k0, int cols) {
  return (q0 + rows <= m.nq) & (k0 + cols <= m.nk) & (k0 >= q0 + rows - 1 - m.lo_off) &
         (k0 + cols - 1 <= q0 + m.hi_off);
}

// Is every (query, key) of that block hidden?
__device__ __forceinline__ bool block_dead(const MaskArgs& m, int q0, int rows, int k0, int cols) {
  return (q0 >= m.nq) | (k0 >= m.nk) | (k0 + cols - 1 < q0 - m.lo_off) |
         (k0 > q0 + rows - 1 + m.hi_off);
}

// Specialise the call to sequence b (its lengths, mask offsets and, for
// varlen, the packed rows it starts at).
__device__ __forceinline__ void bwd_localize(BwdArgs& a, int b) {
  const SeqRows r = seq_localize(a.m, b);
  if (a.m.cu_q) {
    shift_rows<e16>(a.q, r.q0);
    shift_rows<e16>(a.dout, r.q0);
    shift_rows<e16>(a.dq, r.q0);
    shift_rows<e16>(a.k, r.k0);
    shift_rows<e16>(a.v, r.k0);
    shift_rows<e16>(a.dk, r.k0);
    shift_rows<e16>(a.dv, r.k0);
  }
}

}  // namespace
FA_ELEM_NS_END
}  // namespace fa
