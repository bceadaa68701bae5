"""Seeded synthetic inputs shared by the GPU library's callers and the oracle.

This module holds only data generation (random draws, rounding to the
storage type, the workload table).  It contains none of the attention
arithmetic, so both the product path and the oracle-based tests may use it
without sharing any of the method's code.

Inputs follow the workloads the backward is measured on: Q, K, V and dO are
i.i.d. N(0, 1), drawn in that order from numpy's PCG64 with a per-workload
seed, in [B, H, N, d] layout; bf16 workloads round the fp32 draw to bf16
with round-to-nearest-even.
"""

from dataclasses import dataclass, field
import math

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                 # "f32", "bf16" or "f16"
    causal: bool = False
    window_left: int = -1
    window_right: int = -1
    dropout_p: float = 0.0
    seed: int = 0              # generator seed for Q, K, V, dO
    drop_seed: int = 0x5EED    # Philox seed of the dropout mask
    drop_offset: int = 0
    notes: str = field(default="", compare=False)

    @property
    def sm_scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


# The five measured workloads (shapes, masks and dropout as specified for
# the backward's parity and throughput runs).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 64, "f32", seed=1001,
                         notes="non-causal fp32, no dropout"),
    "small_causal_bf16": Workload("small_causal_bf16", 2, 4, 1024, 64, "bf16",
                                  causal=True, seed=1002),
    "train_causal_bf16": Workload("train_causal_bf16", 4, 16, 4096, 128, "bf16",
                                  causal=True, seed=1003,
                                  notes="atomic-dQ and deterministic modes"),
    "window_dropout_bf16": Workload("window_dropout_bf16", 2, 16, 8192, 64, "bf16",
                                    window_left=1023, window_right=1023,
                                    dropout_p=0.1, seed=1004,
                                    notes="two-sided window |i-j| < 1024, dropout 0.1"),
    "long_causal_bf16": Workload("long_causal_bf16", 1, 8, 32768, 128, "bf16",
                                 causal=True, seed=1005),
    "train_causal_f16": Workload("train_causal_f16", 4, 16, 4096, 128, "f16",
                                 causal=True, seed=1006,
                                 notes="the training shape in fp16"),
}


def round_to_bf16_bits(x):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even.

    In 32-bit arithmetic: for every finite or infinite input the bit pattern
    plus 0x8000 stays below 2**32 (only NaN patterns could wrap).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> the same values as fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_tensors(shape, dtype, seed, names=("q", "k", "v", "do"), shapes=None):
    """Draw the named tensors in order from PCG64(seed).

    shapes: optional {name: shape} for tensors whose shape differs from
    `shape` (keys and values of a problem with Nk != Nq, packed varlen
    tensors).  Returns {name: fp32 array of the exact stored values} and,
    for bf16 and fp16, {name + "_bits": uint16 bit patterns} for upload to
    the device.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in names:
        shp = shapes.get(name, shape) if shapes else shape
        x = rng.standard_normal(shp, dtype=np.float64).astype(np.float32)
        if dtype == "bf16":
            bits = round_to_bf16_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
        elif dtype == "f16":
            h = x.astype(np.float16)  # round to nearest even
            out[name + "_bits"] = h.view(np.uint16)
            out[name] = h.astype(np.float32)
        elif dtype == "f32":
            out[name] = x
        else:
            raise ValueError(f"unsupported dtype {dtype!r}")
    return out


def varlen_lengths(count, lo, hi, seed):
    """`count` sequence lengths drawn uniformly from [lo, hi] with PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(lo, hi + 1, size=count)]


def pack_lengths(total, lo, hi, seed):
    """Lengths in [lo, hi] drawn with PCG64(seed) until they fill `total`
    tokens; the last one is cut to fit (a packed batch of a fixed token
    count, as a training step packs documents of mixed length)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out, used = [], 0
    while used < total:
        n = min(int(rng.integers(lo, hi + 1)), total - used)
        out.append(n)
        used += n
    return out


def cumulative(lengths):
    """Offsets [0, l0, l0 + l1, ...] of packed sequences (int32)."""
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def make_workload_inputs(w):
    """The Q, K, V, dO of workload `w` (see make_tensors)."""
    return make_tensors(w.shape, w.dtype, w.seed)
