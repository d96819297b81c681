"""Seeded sweeps of shapes through whole tensor-parallel groups on the GPU,
against the fp64 oracle: N from 1 to 600 tokens (the one-token decode, the
small-batch path and the wide tiles), h and F_i any multiples of 8 (ragged
tiles, k tails and column strips), t from 1 to 4, all three activations, with
and without the output bias; a second sweep at 1 to 129 tokens, where
the backward's input gradients take the split-K kernel (or keep the wide
tiles when the weight gradient cannot hold one split: h < N, F_i < g N); and
a third at 33 to 128 tokens over small weights, where the split-K products
split the token rows into tiles.
The cases are fixed by the seeds below, so every run checks the same ones."""
from __future__ import annotations

import numpy as np
import pytest

from tests.helpers import run_group

pytestmark = pytest.mark.gpu


def _cases(seed=20261202, n=24, wid0=1100, few=False, tiled=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if tiled:
            # 33 to 128 tokens over small weights: the small-batch products
            # split the token rows into 32- or 64-row tiles
            N = int(rng.integers(33, 129))
            h = 8 * int(rng.integers(1, 264))
            t = int(rng.integers(1, 3))
            Fi = 8 * int(rng.integers(1, 200))
            act = ["relu", "gelu", "swiglu"][int(rng.integers(0, 3))]
            bias = bool(rng.integers(0, 2))
            out.append((wid0 + i, N, h, Fi * t, t, act, bias))
            continue
        if few:
            N = int(rng.integers(1, 130))
        else:
            # token counts from each regime: 1, small batches, 65-199, larger
            N = int(rng.choice([1, int(rng.integers(2, 65)), int(rng.integers(65, 200)),
                                int(rng.integers(200, 601))]))
        h = 8 * int(rng.integers(1, 161))
        t = int(rng.integers(1, 5))
        Fi = 8 * int(rng.integers(1, 201))
        act = ["relu", "gelu", "swiglu"][int(rng.integers(0, 3))]
        bias = bool(rng.integers(0, 2))
        out.append((wid0 + i, N, h, Fi * t, t, act, bias))
    return out


CASES = (_cases() + _cases(seed=20261203, n=16, wid0=1140, few=True)
         + _cases(seed=20261205, n=16, wid0=1160, tiled=True))


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[1]}_h{c[2]}_F{c[3]}_t{c[4]}_{c[5]}{'_b' if c[6] else ''}"
                                             for c in CASES])
def test_random_shape_group_matches_oracle(case):
    wid, N, h, F, t, act, bias = case
    run_group(wid, N, h, F, t, act, bias)
