"""Seeded synthetic inputs for the one-shot reduction (bf16 bit patterns).

Both the HIP path's tests and the oracle take their inputs from here; this
module holds none of the reduction's arithmetic. Every array is a numpy
uint16 array of bf16 bit patterns. Floating-point samples are drawn in
float64 with numpy's default_rng, cast to float32, and the bf16 pattern is
the upper 16 bits of that float32 (truncation toward zero: the inputs need a
bf16 value near the sample, not a correctly rounded one).

Workloads (bf16 elements n, W partials):
  1  W=2, [2, 4096]  (n = 8192),     N(0, 1)
  2  W=8, [32, 4096] (n = 131072),   N(0, 1) * 0.1, a fresh own partial per call
  3  W=4, n in {8, 1000, 4096, 65536, 262144}, uniform[-1, 1]
  4  W=8, [8192, 8192] (n = 67108864), N(0, 1)
  5  W=8, [32, 4096] buffers, n = 131071, adversarial mix (see ``adversarial``)

Seeds: recv partial (par, src) of workload c uses 1000*c + 100*par + src; the
own partial of call k uses 1000*c + 500 + k (k = 1, 2, ...).

``bits`` draws raw bf16 patterns, every one of the 65536 equally likely
(so about 1 in 256 is an Inf or a NaN): the limit tests use it for inputs
at the largest size, where every pattern class should appear.
"""
from typing import Dict, List

import numpy as np

WORKLOADS: Dict[int, dict] = {
    1: dict(W=2, n=8192, shape=(2, 4096), dist="normal", scale=1.0),
    2: dict(W=8, n=131072, shape=(32, 4096), dist="normal", scale=0.1),
    3: dict(W=4, ns=(8, 1000, 4096, 65536, 262144), dist="uniform"),
    4: dict(W=8, n=67108864, shape=(8192, 8192), dist="normal", scale=1.0),
    5: dict(W=8, n=131071, shape=(32, 4096), dist="adversarial"),
}

# bf16 patterns used by the adversarial mix
POS_INF, NEG_INF = 0x7F80, 0xFF80
QNAN, NEG_QNAN = 0x7FC0, 0xFFC0
SNAN, NEG_SNAN = 0x7F81, 0xFF81


def f32_to_bf16_trunc(x) -> np.ndarray:
    """Upper half of the float32 pattern of x (x is cast to float32 first)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def normal(seed: int, n: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_trunc(rng.standard_normal(n) * scale)


def uniform(seed: int, n: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_trunc(rng.uniform(lo, hi, n))


def bits(seed: int, n: int) -> np.ndarray:
    """n uniformly random bf16 bit patterns."""
    return np.random.default_rng(seed).integers(0, 1 << 16, size=n, dtype=np.uint16)


def adversarial(seed: int, W: int, n: int) -> List[np.ndarray]:
    """W partials of n elements built to stress the reduction.

    Per partial: half the elements are +-N(0,1)*1e4 and half +-N(0,1)*1e-3
    (cancellation across ranks); then 1 % become random bf16 subnormals
    (exponent 0, random nonzero fraction, random sign) and 0.01 % become
    +-Inf or NaN at seeded positions. Planted columns, the same index in
    every partial: +Inf and -Inf together, NaN with Inf, the signalling NaN
    patterns 0x7F81 / 0xFF81, every partial subnormal, every partial +-0,
    every partial -0, and a large +x / -x pair that cancels exactly.
    """
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(W):
        big = rng.random(n) < 0.5
        mag = np.where(big, 1e4, 1e-3)
        sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
        p = f32_to_bf16_trunc(sign * np.abs(rng.standard_normal(n)) * mag)
        sub = rng.random(n) < 0.01
        frac = rng.integers(1, 0x80, n, dtype=np.uint16)
        sgn = np.where(rng.random(n) < 0.5, 0x8000, 0).astype(np.uint16)
        p = np.where(sub, sgn | frac, p).astype(np.uint16)
        k = max(1, n // 10000)
        pos = rng.choice(n, size=k, replace=False)
        specials = np.array([POS_INF, NEG_INF, QNAN, NEG_QNAN, SNAN, NEG_SNAN], dtype=np.uint16)
        p[pos] = specials[rng.integers(0, len(specials), k)]
        parts.append(p)
    # planted columns (positions spread over the vector part and the tail)
    if n >= 64:
        cols = rng.choice(n - 8, size=24, replace=False)
        cols = np.concatenate([cols, np.arange(n - min(n, 7), n)])
        kinds = ["infinf", "naninf", "snan", "allsub", "allzero", "allnegzero", "cancel"]
        for idx, c in enumerate(cols):
            kind = kinds[idx % len(kinds)]
            if kind == "infinf":
                parts[0][c], parts[W - 1][c] = POS_INF, NEG_INF
            elif kind == "naninf":
                parts[W // 2][c], parts[0][c] = QNAN, NEG_INF
            elif kind == "snan":
                parts[1][c] = SNAN if idx % 2 else NEG_SNAN
            elif kind == "allsub":
                for w in range(W):
                    parts[w][c] = np.uint16((0x8000 if rng.random() < 0.5 else 0) | int(rng.integers(1, 0x80)))
            elif kind == "allzero":
                for w in range(W):
                    parts[w][c] = np.uint16(0x8000 if rng.random() < 0.5 else 0)
            elif kind == "allnegzero":
                for w in range(W):
                    parts[w][c] = np.uint16(0x8000)
            elif kind == "cancel":
                v = int(rng.integers(0x4600, 0x4700))
                for w in range(W):
                    parts[w][c] = np.uint16(0)
                parts[0][c], parts[1][c] = np.uint16(v), np.uint16(v | 0x8000)
    return parts


def _draw(cfg: int, seed: int, n: int) -> np.ndarray:
    w = WORKLOADS[cfg]
    if w["dist"] == "normal":
        return normal(seed, n, w["scale"])
    if w["dist"] == "uniform":
        return uniform(seed, n)
    raise ValueError(f"workload {cfg} has no single-partial draw")


def recv_partials(cfg: int, par: int, n: int, W: int = None) -> List[np.ndarray]:
    """The W partials of parity `par` (index = source rank). The entry at this
    rank's own index is a valid partial too; callers that model a peer set
    use it or ignore it."""
    W = W or WORKLOADS[cfg]["W"]
    if WORKLOADS[cfg]["dist"] == "adversarial":
        return adversarial(1000 * cfg + 100 * par, W, n)
    return [_draw(cfg, 1000 * cfg + 100 * par + src, n) for src in range(W)]


def own_partial(cfg: int, call: int, n: int) -> np.ndarray:
    """This rank's partial for call number `call` (1-based)."""
    if WORKLOADS[cfg]["dist"] == "adversarial":
        return adversarial(1000 * cfg + 500 + call, WORKLOADS[cfg]["W"], n)[0]
    return _draw(cfg, 1000 * cfg + 500 + call, n)
