"""Seeded synthetic attention inputs (bf16 bit patterns as uint16 arrays).

Shared by the oracle-side tests and the GPU-side tests and benchmark; it holds
none of the attention or quantization arithmetic, only random numbers:

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", 2014) read as a counter-based generator: the i-th 64-bit word of
  a stream with key k is mix(k + (i + 1) * 0x9E3779B97F4A7C15);
* uniforms u = (word >> 11 + 1) * 2^-53 in (0, 1];
* Box-Muller: n = sqrt(-2 ln u1) * cos(2 pi u2);
* float32 -> bf16 with round-to-nearest-even.

The workloads mirror the shapes and value structure of the pages' synthetic
harnesses (see ``workload``): per-channel K means, K outliers, low-rank peaked
Q/K for video-DiT-like attention, grouped-query heads and packed documents with
log-uniform lengths.
"""
from __future__ import annotations

import math

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> np.uint64:
    """Key of an independent stream: mix(seed + stream * 0xD1B54A32D192ED03)."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + np.uint64(stream) * np.uint64(0xD1B54A32D192ED03)
    return _mix(np.array([z], dtype=np.uint64))[0]


def words(key: np.uint64, start: int, n: int) -> np.ndarray:
    """Words start .. start+n-1 of the stream with the given key."""
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + idx * _GAMMA)


def uniform(seed: int, stream: int, n: int) -> np.ndarray:
    """n uniforms in (0, 1] (float64)."""
    key = stream_key(seed, stream)
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        w = words(key, s, min(_CHUNK, n - s))
        out[s:s + len(w)] = ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    return out


def normal(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard normals (float64) by Box-Muller over word pairs (2i, 2i+1)."""
    key = stream_key(seed, stream)
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        w = words(key, 2 * s, 2 * m)
        u = ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        out[s:s + m] = np.sqrt(-2.0 * np.log(u[0::2])) * np.cos(2.0 * math.pi * u[1::2])
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16(x: np.ndarray) -> np.ndarray:
    return f32_to_bf16(x.astype(np.float32))


def _outliers(x: np.ndarray, seed: int, stream: int, frac: float, factor: float) -> None:
    """Multiply round(frac * size) distinct, uniformly chosen entries by factor
    (first distinct indices of a uniform index stream)."""
    flat = x.reshape(-1)
    k = int(round(frac * flat.size))
    if k == 0:
        return
    u = uniform(seed, stream, 2 * k + 64)
    cand = np.minimum((u * flat.size).astype(np.int64), flat.size - 1)
    _, first = np.unique(cand, return_index=True)
    chosen = cand[np.sort(first)][:k]
    if chosen.size != k:
        raise RuntimeError("outlier draw produced too few distinct indices")
    flat[chosen] *= factor


def doc_lengths(seed: int, total: int, lo: int, hi: int) -> np.ndarray:
    """Document lengths round(exp(U(ln lo, ln hi))) drawn until the next draw
    would pass ``total``; the last document takes the remainder."""
    u = uniform(seed, 900, 4096)
    lens, acc = [], 0
    for ui in u:
        L = int(round(math.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * ui)))
        if acc + L > total:
            break
        lens.append(L)
        acc += L
    if acc < total:
        lens.append(total - acc)
    return np.array(lens, dtype=np.int64)


def gaussian(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    return (normal(seed, stream, int(np.prod(shape))) * std).reshape(shape)


def make_inputs(kind: str, B: int, Hq: int, Hkv: int, N: int, d: int = 128, seed: int = 0,
                total_tokens: int | None = None):
    """Synthetic Q, K, V as bf16 bit patterns ([B,Hq,N,d], [B,Hkv,N,d], [B,Hkv,N,d]).

    kind:
      "kmean"    Q, V ~ N(0,1); K ~ N(0,1) plus a per-channel mean mu_c ~ N(0, var 2)
                 shared by all tokens of a head
      "kmean_outlier"  as "kmean" and 0.1% of K entries multiplied by 20
      "lowrank"  per head W ~ N(0,1)^{16 x d} shared by Q and K, U_q, U_k ~ N(0,1)^{N x 16};
                 Q = 1.5 U_q W / 4 + eps_q, K likewise, eps ~ N(0, var 0.5); V ~ N(0,1)
      "outlier"  Q, K, V ~ N(0,1), 0.1% of K entries multiplied by 20
      "plain"    Q, K, V ~ N(0,1)
    Returns dict(q, k, v) of uint16 arrays.
    """
    q = gaussian(seed, 1, (B, Hq, N, d))
    v = gaussian(seed, 3, (B, Hkv, N, d))
    if kind == "lowrank":
        r = 16
        W = gaussian(seed, 10, (B, Hkv, r, d))
        Uq = gaussian(seed, 11, (B, Hq, N, r))
        Uk = gaussian(seed, 12, (B, Hkv, N, r))
        grp = Hq // Hkv
        Wq = np.repeat(W, grp, axis=1)
        q = 1.5 * np.matmul(Uq, Wq) / 4.0 + gaussian(seed, 13, (B, Hq, N, d), math.sqrt(0.5))
        k = 1.5 * np.matmul(Uk, W) / 4.0 + gaussian(seed, 14, (B, Hkv, N, d), math.sqrt(0.5))
    else:
        k = gaussian(seed, 2, (B, Hkv, N, d))
        if kind in ("kmean", "kmean_outlier"):
            mu = gaussian(seed, 4, (B, Hkv, 1, d), math.sqrt(2.0))
            k = k + mu
        if kind in ("kmean_outlier", "outlier"):
            _outliers(k, seed, 5, 0.001, 20.0)
    return {"q": _bf16(q), "k": _bf16(k), "v": _bf16(v)}


# Workloads of the five measured configurations, full size and a reduced size
# that the oracle finishes in seconds while still spanning several tiles.
WORKLOADS = {
    "c1_single_head": dict(B=1, Hq=1, Hkv=1, N=1024, kind="kmean", causal=False),
    "c2_mha_4k": dict(B=2, Hq=16, Hkv=16, N=4096, kind="kmean_outlier", causal=False),
    "c3_video_dit_32k": dict(B=1, Hq=24, Hkv=24, N=32768, kind="lowrank", causal=False),
    "c4_gqa_causal_32k": dict(B=1, Hq=32, Hkv=8, N=32768, kind="kmean", causal=True),
    "c5_varlen_causal_64k": dict(B=1, Hq=16, Hkv=16, N=65536, kind="outlier", causal=True,
                                 varlen=(512, 16384)),
}


def workload(name: str, seed: int = 0, N: int | None = None, H: int | None = None):
    """Inputs of a named workload; N and H may shrink it (GQA ratio kept)."""
    w = dict(WORKLOADS[name])
    if N is not None:
        w["N"] = N
    if H is not None:
        ratio = w["Hq"] // w["Hkv"]
        w["Hq"] = H
        w["Hkv"] = max(1, H // ratio)
    out = make_inputs(w["kind"], w["B"], w["Hq"], w["Hkv"], w["N"], 128, seed)
    out.update(w)
    if "varlen" in w:
        lo, hi = w["varlen"]
        if w["N"] < hi:  # reduced size: shrink the length range with the total
            f = w["N"] / WORKLOADS[name]["N"]
            lo, hi = max(16, int(lo * f)), max(32, int(hi * f))
        lens = doc_lengths(seed, w["N"], lo, hi)
        out["doc_off"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    else:
        out["doc_off"] = None
    return out
