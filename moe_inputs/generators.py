"""Workload table and seeded generators (no layer arithmetic here)."""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Stream ids, in the fixed order the workloads are drawn.
S_X, S_WR, S_WG, S_WU, S_WD, S_DY, S_ROUTE, S_GATE = range(8)
_W_STREAM = {"w_gate": S_WG, "w_up": S_WU, "w_down": S_WD}

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    """One MoE-layer shape: T tokens, d model width, E experts, top-k, d_ff f."""

    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    dtype: str  # "f32", "bf16" or "mxfp8" (bf16 master values, quantised in-step)
    routing: str  # "learned" (router GEMM + softmax top-k), "zipf", "balanced"
    zipf_s: float = 1.2

    @property
    def S(self) -> int:
        return self.T * self.k

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        return {"workload": self.name, "T": self.T, "d_model": self.d, "experts": self.E,
                "top_k": self.k, "d_ff": self.f, "dtype": self.dtype, "routing": self.routing}


WORKLOADS = {
    # Tiny fp32 layer used for exhaustive parity at full size.
    "tiny_f32": Workload("tiny_f32", 256, 64, 8, 4, 128, "f32", "learned"),
    # bf16 layer with 8 experts (the headline throughput workload).
    "bf16_e8": Workload("bf16_e8", 8192, 2048, 8, 4, 1024, "bf16", "learned"),
    # Same active compute spread over 128 experts.
    "bf16_e128": Workload("bf16_e128", 8192, 2048, 128, 4, 1024, "bf16", "learned"),
    # Skewed load: Zipf(1.2) expert popularity, random (not learned) routing.
    "bf16_zipf": Workload("bf16_zipf", 16384, 4096, 128, 4, 1536, "bf16", "zipf"),
    # MXFP8 layer with uniformly balanced random routing.
    "mxfp8_balanced": Workload("mxfp8_balanced", 32768, 4096, 128, 4, 1536, "mxfp8", "balanced"),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    Inputs here are always finite, so the NaN case is not handled.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 array whose values are the bf16 (RNE) roundings of ``a``."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.astype(np.float32) if dtype == "f32" else bf16_round(a)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def expert_weight(wl: Workload, which: str, e: int, seed: int = 0) -> np.ndarray:
    """One expert's weight matrix: w_gate/w_up are [d, f], w_down is [f, d]."""
    shape = (wl.f, wl.d) if which == "w_down" else (wl.d, wl.f)
    return _store(_normal(_rng(seed, _W_STREAM[which], e), shape, WEIGHT_STD), wl.dtype)


def _all_experts(wl: Workload, which: str, seed: int, threads: int) -> np.ndarray:
    shape = (wl.f, wl.d) if which == "w_down" else (wl.d, wl.f)
    out = np.empty((wl.E,) + shape, dtype=np.float32)

    def one(e):
        out[e] = expert_weight(wl, which, e, seed)

    if threads > 1 and wl.E > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(wl.E)))
    else:
        for e in range(wl.E):
            one(e)
    return out


def zipf_routing(T: int, E: int, k: int, s: float, seed: int = 0, popularity=None):
    """k distinct experts per token drawn without replacement, P(expert r-1) ~ r^-s.

    Sampling without replacement uses the Gumbel-top-k construction: add
    independent Gumbel noise to the log-popularities and keep the k largest;
    this is the same law as k sequential draws renormalised after each one.
    Slot order is by decreasing perturbed key. ``popularity`` may override
    the Zipf weights (entries of 0 make an expert never chosen).
    Gates are independent U(0,1) per slot divided by the token's sum.
    """
    if popularity is None:
        popularity = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    popularity = np.asarray(popularity, dtype=np.float64)
    if int((popularity > 0).sum()) < k:
        raise ValueError("fewer than k experts have non-zero popularity")
    with np.errstate(divide="ignore"):
        logp = np.log(popularity / popularity.sum())
    keys = _rng(seed, S_ROUTE).gumbel(size=(T, E)) + logp[None, :]
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    return idx, _uniform_gates(T, k, seed)


def balanced_routing(T: int, E: int, k: int, seed: int = 0):
    """Uniform balanced random routing: each expert receives exactly T*k/E rows.

    Tokens are dealt in blocks of E/k: each block gets a fresh random
    permutation of all E experts, cut into consecutive groups of k.
    """
    if E % k or T % (E // k):
        raise ValueError("balanced routing needs k | E and (E/k) | T")
    rng = _rng(seed, S_ROUTE)
    blocks = T // (E // k)
    idx = np.stack([rng.permutation(E) for _ in range(blocks)]).reshape(T, k).astype(np.int32)
    return idx, _uniform_gates(T, k, seed)


def _uniform_gates(T: int, k: int, seed: int) -> np.ndarray:
    u = _rng(seed, S_GATE).uniform(size=(T, k))
    return (u / u.sum(axis=1, keepdims=True)).astype(np.float32)


def make_inputs(wl: Workload, seed: int = 0, weights: bool = True, threads: int = 8,
                popularity=None) -> dict:
    """All inputs of one layer forward+backward as fp32 numpy arrays.

    For bf16/mxfp8 workloads every floating value is exactly representable in
    bf16. Keys: x [T,d], dy [T,d], w_gate [E,d,f], w_up [E,d,f], w_down [E,f,d],
    and either w_router [d,E] (learned routing) or topk_idx [T,k] int32 and
    topk_gate [T,k] fp32 (random routing).
    """
    out = {
        "x": _store(_normal(_rng(seed, S_X), (wl.T, wl.d), 1.0), wl.dtype),
        "dy": _store(_normal(_rng(seed, S_DY), (wl.T, wl.d), 1.0), wl.dtype),
    }
    if wl.routing == "learned":
        out["w_router"] = _store(_normal(_rng(seed, S_WR), (wl.d, wl.E), WEIGHT_STD), wl.dtype)
    elif wl.routing == "zipf":
        out["topk_idx"], out["topk_gate"] = zipf_routing(wl.T, wl.E, wl.k, wl.zipf_s, seed, popularity)
    elif wl.routing == "balanced":
        out["topk_idx"], out["topk_gate"] = balanced_routing(wl.T, wl.E, wl.k, seed)
    else:
        raise ValueError(wl.routing)
    if weights:
        for w in ("w_gate", "w_up", "w_down"):
            out[w] = _all_experts(wl, w, seed, threads)
    return out
