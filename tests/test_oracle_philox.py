"""Pins of the oracle's Philox4x32-10 and dropout mask.

Two independent library implementations of Philox4x32-10 serve as witnesses:
PyTorch's header-only engine (compiled with g++) and rocRAND's (compiled
with hipcc for the host).  Both are built and run at test time; no output of
theirs is stored.  Their stream (seed, subsequence, offset) places the seed
in the key and (offset, subsequence) in the counter words, which is the
mapping the dropout mask uses with subsequence = (b<<48)|(h<<32)|(i<<16)|j0,
j0 = 16 m or 16 m + 4: the block serves keys j0 .. j0 + 3 and j0 + 8 .. j0 + 11
at positions 0 .. 7, position q taking the 16-bit half q mod 2 (low half
first) of word q div 2.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _torch_include():
    import torch
    return os.path.join(os.path.dirname(torch.__file__), "include")


def _build(tmp_path_factory, which):
    src = os.path.join(HERE, "witness", f"philox_{which}.cpp")
    out = str(tmp_path_factory.mktemp("witness") / which)
    if which == "torch":
        cmd = ["g++", "-O1", "-std=c++17", "-I", _torch_include(), src, "-o", out]
    else:
        hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
        if not os.path.exists(hipcc):
            pytest.skip("hipcc not available for the rocRAND witness")
        cmd = [hipcc, "-O1", "-std=c++17", src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


@pytest.fixture(scope="module", params=["torch", "rocrand"])
def witness(request, tmp_path_factory):
    return _build(tmp_path_factory, request.param)


def _cases():
    rng = np.random.default_rng(2024)
    seeds = [0, 1, 0x5EED, 0xFFFFFFFF, 1 << 32, (1 << 64) - 1]
    seeds += [int(x) for x in rng.integers(0, 2**63, 4)]
    offsets = [0, 1, 0xFFFFFFFF, 1 << 32, (1 << 40) + 12345]
    coords = [(0, 0, 0, 0), (65535, 65535, 65535, 65524), (1, 2, 3, 16), (3, 15, 8191, 7008),
              (65535, 65535, 65535, 65535), (1, 2, 3, 5), (1, 2, 3, 4), (7, 8, 9, 65520)]
    coords += [tuple(int(x) for x in rng.integers(0, 65536, 4)) for _ in range(6)]
    coords += [tuple(int(x) for x in rng.integers(0, 65536, 3)) + (4 * int(rng.integers(0, 16384)),)
               for _ in range(6)]
    cases = []
    for s in seeds:
        for o in offsets:
            for c in coords:
                cases.append((s, o) + c)
    return cases


def _run(witness, cases):
    lines = []
    for seed, off, b, h, i, j in cases:
        sub = (b << 48) | (h << 32) | (i << 16) | j
        lines.append(f"{seed} {sub} {off}")
    res = subprocess.run([witness], input="\n".join(lines) + "\n", capture_output=True,
                         text=True, check=True)
    return [[int(w, 16) for w in line.split()] for line in res.stdout.strip().splitlines()]


def test_block_function_matches_witness(witness):
    cases = _cases()
    expect = _run(witness, cases)
    assert len(expect) == len(cases)
    for (seed, off, b, h, i, j), words in zip(cases, expect):
        counter = (off & 0xFFFFFFFF, off >> 32, (i << 16) | j, (b << 16) | h)
        key = (seed & 0xFFFFFFFF, seed >> 32)
        got = [int(w) for w in oracle.philox4x32_10(counter, key)]
        assert got == words, (seed, off, b, h, i, j)
        if j % 16 in (0, 4):
            # the block of keys j .. j + 3, j + 8 .. j + 11: position q draws
            # the 16-bit half q mod 2 (low first) of word q div 2
            cols = [j + q for q in range(4)] + [j + 8 + q for q in range(4)]
            x = oracle.dropout_uniform_bits(seed, off, b, h, [i], cols)[0]
            halves = [(w >> (16 * k)) & 0xFFFF for w in words for k in range(2)]
            assert [int(v) for v in x] == halves, (seed, off, b, h, i, j)


def test_keep_threshold_is_exact():
    assert oracle.keep_threshold(0.0) == 0
    assert oracle.keep_threshold(0.1) == 6554               # ceil(0.1 * 2**16)
    assert oracle.keep_threshold(0.5) == 1 << 15
    assert oracle.keep_threshold(1 - 2**-16) == 0xFFFF
    with pytest.raises(ValueError):
        oracle.keep_threshold(1.0)
    with pytest.raises(ValueError):
        oracle.keep_threshold(1 - 2**-17)                   # T would be 2**16
    # x >= T  <=>  x / 2**16 >= p, checked at the boundary
    t = oracle.keep_threshold(0.1)
    assert (t - 1) / 2**16 < 0.1 <= t / 2**16


def test_keep_fraction_and_uniformity():
    n = 1024
    x = oracle.dropout_uniform_bits(0x5EED, 0, 1, 3, np.arange(n), np.arange(n)).ravel()
    keep = oracle.dropout_keep(0x5EED, 0, 1, 3, np.arange(n), np.arange(n), 0.1).ravel()
    frac = keep.mean()
    sigma = np.sqrt(0.1 * 0.9 / keep.size)
    assert abs(frac - 0.9) < 6 * sigma
    # chi-square of the top byte of the 16-bit draw against uniform (255
    # dof; 6 sigma ~ 391), and of the low byte
    counts = np.bincount((x >> 8).astype(np.int64), minlength=256)
    expected = x.size / 256
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)
    counts = np.bincount((x & 0xFF).astype(np.int64), minlength=256)
    expected = x.size / 256
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)


def test_mask_changes_with_offset_and_head():
    idx = np.arange(256)
    a = oracle.dropout_keep(0x5EED, 0, 0, 0, idx, idx, 0.1)
    b = oracle.dropout_keep(0x5EED, 1, 0, 0, idx, idx, 0.1)
    c = oracle.dropout_keep(0x5EED, 0, 0, 1, idx, idx, 0.1)
    assert (a != b).mean() > 0.1 and (a != c).mean() > 0.1


def test_words_of_one_block_serve_eight_keys():
    """Keys 16 m + 4 t + (0..3) and 16 m + 8 + 4 t + (0..3) of a row (t = 0, 1)
    share one block, two per word (low half first); every key of the row is
    served by exactly one block position."""
    rows = np.arange(5)
    cols = np.arange(64)
    x = oracle.dropout_uniform_bits(0x5EED, 7, 2, 9, rows, cols)
    for i in rows:
        seen = np.zeros(64, dtype=int)
        for m in range(4):
            for t in range(2):
                j0 = 16 * m + 4 * t
                counter = (7, 0, (int(i) << 16) | j0, (2 << 16) | 9)
                words = [int(w) for w in oracle.philox4x32_10(counter, (0x5EED, 0))]
                halves = [w & 0xFFFF if k % 2 == 0 else w >> 16 for w in words for k in range(2)]
                keys = [j0 + q for q in range(4)] + [j0 + 8 + q for q in range(4)]
                assert [int(v) for v in x[i, keys]] == halves
                seen[keys] += 1
        assert (seen == 1).all()
