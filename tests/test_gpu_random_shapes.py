"""Randomised prefill parity: seeded random shapes, windows, rotary dims and positions
through both layer kinds, against the fp64 oracle.

Each case draws the batch, the sequence length (1 .. 1100: one to eighteen 64-key tiles
with a ragged tail), the head group (1, 2, 4, 8), the head dim (64, 128), the rotary dim
(0, the model's 2 floor(0.33 d / 2) or any even value up to 64), the window and the
position offset, so that tile boundaries, masked diagonal and band-edge tiles and the
windows' edges fall at places no hand-written case chose. Every fourth case takes the
model's head shape (d = 128, four query heads per KV head, rotary 42, window <= 128), the
shape the streaming SWA kernel serves. The global layer runs with and without the K~
workspace. bf16 inputs, max-abs error 2e-2 against the oracle over every row.
"""

import numpy as np
import pytest

from tests.gpu_util import TOL_BF16
from tests.test_gpu_prefill import _check, _inputs

pytestmark = pytest.mark.gpu


def _cases(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        model = i % 4 == 3
        d = 128 if model else int(rng.choice([64, 128]))
        group = 4 if model else int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2]))
        B = int(rng.choice([1, 2]))
        T = int(rng.integers(1, 1101))
        if model:
            r = 42
            W = int(rng.integers(1, 129))
        else:
            r = int(rng.choice([0, 2 * int(0.33 * d / 2), 2 * int(rng.integers(1, 33))]))
            W = int(rng.integers(1, 400))
        pos = int(rng.integers(0, 100_000))
        cases.append((i, B, T, hkv * group, hkv, d, r, W, pos))
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_shapes_both_layers(case):
    i, B, T, Hq, Hkv, d, r, W, pos = case
    q, k, v, g, wq, wk = _inputs(B, T, Hq, Hkv, d, "bf16", 9000 + 10 * i)
    _check("swa", q, k, v, g, wq, wk, window=W, rdim=r, pos_offset=pos, tol=TOL_BF16)
    _check("global", q, k, v, None, wq, wk, rdim=r, pos_offset=pos, tol=TOL_BF16)
    _check("global", q, k, v, None, wq, wk, rdim=r, pos_offset=pos, tol=TOL_BF16,
           workspace=None)
