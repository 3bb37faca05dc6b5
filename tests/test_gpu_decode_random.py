"""A seeded sweep of split-key decode configurations against the oracle's split decode:
every P mode, both QK4PV8 Q/K formats, grouped-query ratios and newest-row counts up
to the 32 packed columns (both column forms), odd history lengths and a ragged history
length per request.  The fragile-row share is reported, not capped."""
import numpy as np
import pytest

from helpers import gpu_available
from test_gpu_decode import run_decode

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N_DRAWS = 24


def _draw(i):
    rng = np.random.default_rng(20261204 + i)
    pm = ["direct", "pnq", "two_level", "fp8"][int(rng.integers(4))]
    qfmt = ["nvfp4", "mxfp4"][int(rng.integers(2))] if pm == "fp8" else None
    Hkv = int(rng.choice([1, 2, 4]))
    gsz = int(rng.choice([1, 2, 4, 8]))
    R = int(rng.integers(1, 5))
    while gsz * R > 32:
        R -= 1
    B = int(rng.integers(1, 4))
    N = int(rng.integers(R, 2601))
    kv_len = [int(x) for x in rng.integers(R, N + 1, size=B)]
    return dict(pm=pm, qfmt=qfmt, B=B, Hq=Hkv * gsz, Hkv=Hkv, R=R, N=N, kv_len=kv_len, seed=2000 + i)


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_decode_random_configuration(i):
    c = _draw(i)
    print(f"random decode {i}: {c}", flush=True)
    run_decode(c["pm"], c["B"], c["Hq"], c["Hkv"], c["R"], c["N"], c["kv_len"], c["seed"], qfmt=c["qfmt"], cap=None)
