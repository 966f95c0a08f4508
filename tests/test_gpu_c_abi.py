"""GPU: a C program drives libpa.so through include/pa.h alone.

tests/c_abi_decode.c (built by __graft_entry__.build() with gcc against the
header, libpa.so and the HIP runtime; no Python in the loop) creates a paged
fp32 pool over its own hipMalloc'd cache, admits a batch, appends every token
but the last with pa_reserve + pa_append_kv, reserves the step's token, and
decodes two layers: layer 0 with pa_append_decode, layer 1 with
pa_decode_plan + pa_append_decode_planned.  This test writes the seeded
inputs, runs the program and checks its outputs against the oracle's fp64
attention over the same logical rows (fp32 cache: 1e-5 absolute).  The batch
(64 sequences, 2 KV heads, 64-token partitions of contexts up to 1100 tokens)
makes a split launch large enough to run from a work plan.
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import attention as A

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_decode")
F32_ABS = 1e-5


def test_c_program_decodes_two_layers_like_the_oracle(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert os.path.exists(EXE), "tests/c_abi_decode is built by __graft_entry__.build()"
    rng = np.random.default_rng(2417)
    B, Hq, Hkv, D, BS, layers, S, pt = 64, 4, 2, 64, 16, 2, 1152, 64
    lens = rng.integers(1, 1101, B).astype(np.int32)
    lens[:5] = [1, 16, 17, 64, 1100]        # one token, block and partition edges, the longest
    nb = int(sum(-(-int(x) // BS) for x in lens)) + 8
    order = rng.permutation(nb).astype(np.int32)
    rows = int(lens.sum())
    q = rng.standard_normal((layers, B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((layers, rows, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((layers, rows, Hkv, D)).astype(np.float32)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([B, Hq, Hkv, D, BS, nb, layers, S, pt], dtype=np.int32).tobytes())
        for arr in (lens, order, q, k, v):
            f.write(np.ascontiguousarray(arr).tobytes())
    print(f"c_abi_decode: B {B} Hq {Hq} Hkv {Hkv} D {D} BS {BS} NB {nb} pt {pt}", flush=True)
    res = subprocess.run([EXE, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]
    raw = np.fromfile(outp, dtype=np.uint8)
    planned = int(raw[:4].view(np.int32)[0])
    got_lens = raw[4:4 + 4 * B].view(np.int32)
    out = raw[4 + 4 * B:].view(np.float32).reshape(layers, B, Hq, D)
    assert planned == 1                       # 64 x 2 x 18 partitions: the launch runs from a plan
    assert np.array_equal(got_lens, lens)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    first = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for layer in range(layers):
        for s in range(B):
            a, n = int(first[s]), int(lens[s])
            ref = A.attend(q[layer, s].astype(np.float64), k[layer, a:a + n].astype(np.float64),
                           v[layer, a:a + n].astype(np.float64), scale)
            err = float(np.max(np.abs(out[layer, s].astype(np.float64) - ref)))
            assert err <= F32_ABS, (layer, s, n, err)
