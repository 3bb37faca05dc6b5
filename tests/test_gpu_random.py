"""A seeded sweep of forward configurations against the oracle, beyond the fixed cases:
odd lengths, random document splits, grouped-query ratios, causal or not, every operand
route of the ping-pong and single-buffer kernels, and the causally safe V form where
the route has one.  Each draw is a small problem compared element by element under the
usual bound (2e-3 max|O| + the flip budget); the fragile-row share is reported, not
capped, since a draw may land on a short row with many threshold decisions."""
import numpy as np
import pytest

from helpers import TOL, gpu_available, record_parity, run_case
from test_gpu_fwd import ROUTES

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N_DRAWS = 48


def _draw(i):
    rng = np.random.default_rng(20261203 + i)
    route = sorted(ROUTES)[int(rng.integers(len(ROUTES)))]
    q, v, pm, pf = ROUTES[route]
    docs = rng.random() < 0.4
    B = 1 if docs else int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    N = int(rng.integers(1, 1101))
    causal = bool(rng.random() < 0.6)
    doc_off = None
    if docs and N >= 2:
        nd = int(rng.integers(1, min(6, N) + 1))
        cuts = np.sort(rng.choice(np.arange(1, N), size=nd - 1, replace=False)) if nd > 1 else np.array([], int)
        doc_off = np.concatenate([[0], cuts, [N]]).astype(np.int32)
    # the per-key V form: causal, a 4-bit V with E8M0 scales per 32 keys (the ping-pong kernel)
    safe = causal and v.startswith("mxfp4") and pm != "fp8" and bool(rng.random() < 0.5)
    kind = ["kmean", "outlier", "plain"][int(rng.integers(3))]
    return dict(route=route, q=q, v=v, pm=pm, pf=pf, B=B, Hq=Hq, Hkv=Hkv, N=N, causal=causal, doc_off=doc_off,
                safe=safe, kind=kind, seed=1000 + i)


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_fwd_random_configuration(i):
    c = _draw(i)
    name = (f"random {i}: {c['route']} B{c['B']} Hq{c['Hq']} Hkv{c['Hkv']} N{c['N']} causal={c['causal']} "
            f"docs={None if c['doc_off'] is None else len(c['doc_off']) - 1} safe={c['safe']} {c['kind']}")
    print(name, flush=True)
    res = run_case(c["q"], c["v"], c["pm"], c["pf"], c["B"], c["Hq"], c["Hkv"], c["N"], causal=c["causal"],
                   kind=c["kind"], seed=c["seed"], doc_off=c["doc_off"], safe=c["safe"])
    print(f"{name}: max err/bound {res['ratio']:.3f}, fragile rows {res['n_fragile']}", flush=True)
    assert np.all(np.isfinite(res["O_gpu"]))
    record_parity(name, res["ratio"], res["fb"] / (TOL * max(res["amax"], 1e-30)), None)
    assert res["ratio"] <= 1.0, name
