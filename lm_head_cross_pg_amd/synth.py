"""Seeded synthetic inputs for the tied LM head + softcap cross-entropy -> bits-per-byte path.

This module holds no arithmetic of the method itself: it only draws arrays. It serves both the
HIP path (benchmarks, smoke run) and the CPU oracle (tests); neither of those imports the other.

The challenge scores a small GPT on FineWeb validation text, which is not available here. The
stand-in keeps what the head sees of that workload:

* model width d = 512 and vocabularies of 1024 / 8192 BPE entries
  (HYDRA Golf site, "Core GPT"; parameter-golf README leaderboard, "Naive Baseline" row),
* sequences of 2048 tokens (README leaderboard, "2048 seq length" row), so T = batch x 2048 rows,
* tied input/output embeddings (trios issue, "Tied embeddings" row of the approach table),
* Zipf-distributed next-token ids (a BPE vocabulary is ranked by frequency),
* UTF-8 byte lengths per vocabulary entry (the metric counts bytes, tproger article "Правила и
  метрика"), drawn from a shifted, clipped Poisson law,
* sliding-window scoring at stride 64 (README leaderboard, "Sliding Window Eval" row) as a mask,
  with BOS tokens (id 0, zero bytes) at geometric gaps.

Every array is drawn from ``numpy.random.default_rng([seed, stream])`` in the fixed order
hidden, embedding, targets, byte lengths, mask/BOS. bf16 arrays are produced by round-to-nearest-
even from float32 and are stored as their uint16 bit patterns, so the GPU run and the oracle read
exactly the same values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "make_inputs", "bf16_bits", "bf16_to_f64", "as_f64",
    "stride_mask", "zipf_pmf", "make_stream", "window_hidden",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value distribution of one synthetic workload."""
    name: str
    stream: int            # second word of the generator seed
    T: int                 # token rows (batch x sequence, flattened)
    D: int                 # hidden width
    V: int                 # vocabulary size
    dtype: str             # "bf16" or "f32" for hidden and embedding
    softcap: float = 30.0
    hidden: str = "unit_rms"   # "normal" (N(0,1)) or "unit_rms" (N(0,1) rows rescaled to RMS 1)
    hidden_scale: float = 1.0  # multiplies hidden after normalisation (stress shape only)
    embed_std: float = 0.02
    targets: str = "zipf"      # "uniform" or "zipf"
    zipf_s: float = 1.1
    bytes_law: str = "poisson"  # "uniform" or "poisson"
    bytes_lo: int = 1
    bytes_hi: int = 16
    poisson_lam: float = 2.7
    seq_len: int = 2048
    stride: Optional[int] = None    # if set: score only the last `stride` rows of each window
    bos_rate: Optional[float] = None  # if set: id 0 is BOS, placed at geometric gaps

    @property
    def scored_rows(self) -> int:
        if self.stride is None:
            return self.T
        return (self.T // self.seq_len) * self.stride


def _w(**kw) -> Workload:
    return Workload(**kw)


# The five measured workloads plus two test-only shapes. Keys name the workload by what it is.
WORKLOADS = {
    # tiny fp32 forward, all rows scored, uniform targets, 1..8 bytes per entry
    "tiny_f32": _w(name="tiny_f32", stream=0, T=256, D=64, V=512, dtype="f32", hidden="normal",
                   targets="uniform", bytes_law="uniform", bytes_lo=1, bytes_hi=8),
    # baseline-vocab forward: 4 x 2048 rows, V = 1024, 1..12 bytes (mean 2.5)
    "fwd_v1024": _w(name="fwd_v1024", stream=1, T=8192, D=512, V=1024, dtype="bf16",
                    bytes_hi=12, poisson_lam=1.5),
    # main forward: 32 x 2048 rows, V = 8192, 1..16 bytes (mean 3.7)
    "fwd_v8192": _w(name="fwd_v8192", stream=2, T=65536, D=512, V=8192, dtype="bf16",
                    bytes_hi=16, poisson_lam=2.7),
    # masked sliding-window forward: last 64 rows of every 2048 window scored; BOS at ~1/700
    "masked_stride64": _w(name="masked_stride64", stream=3, T=65536, D=512, V=8192, dtype="bf16",
                          bytes_hi=16, poisson_lam=2.7, stride=64, bos_rate=1.0 / 700.0),
    # training forward + backward, mean-reduced loss over every row
    "train_v8192": _w(name="train_v8192", stream=4, T=65536, D=512, V=8192, dtype="bf16",
                      bytes_hi=16, poisson_lam=2.7),
    # finite-difference shape for the gradient pins (oracle only)
    "fd": _w(name="fd", stream=5, T=64, D=32, V=128, dtype="f32", hidden="normal",
             targets="uniform", bytes_law="uniform", bytes_lo=1, bytes_hi=8),
    # softcap stress: hidden scaled so that |z| reaches several c and tanh curvature matters
    "stress": _w(name="stress", stream=6, T=256, D=64, V=512, dtype="bf16", hidden="normal",
                 hidden_scale=280.0, targets="uniform", bytes_law="uniform", bytes_lo=1,
                 bytes_hi=8),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input array (bf16 bits or float32) -> float64, exactly."""
    return bf16_to_f64(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float64)


def zipf_pmf(n: int, s: float) -> np.ndarray:
    """Probabilities of ranks 1..n under a Zipf law truncated to n ranks."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def _zipf_draw(rng: np.random.Generator, size: int, n: int, s: float) -> np.ndarray:
    """Ranks 1..n drawn by inverse CDF; returned as 0-based rank indices."""
    cdf = np.cumsum(zipf_pmf(n, s))
    cdf[-1] = 1.0
    return np.searchsorted(cdf, rng.random(size), side="right").astype(np.int64)


def stride_mask(T: int, seq_len: int, stride: int) -> np.ndarray:
    """uint8[T]: 1 on the last `stride` rows of every `seq_len` window, else 0."""
    m = np.zeros(T, dtype=np.uint8)
    pos = np.arange(T) % seq_len
    m[pos >= seq_len - stride] = 1
    return m


def make_inputs(w: Workload | str, seed: int = 0, T: Optional[int] = None) -> dict:
    """Draw one workload's inputs.

    Returns a dict with ``hidden [T,D]`` and ``embed [V,D]`` (uint16 bf16 bits or float32),
    ``target int32[T]``, ``byte_len int32[V]``, ``mask uint8[T]`` or None, plus the shape and
    ``softcap``. ``T`` may override the row count (same distribution, fewer rows).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    T = w.T if T is None else int(T)
    D, V = w.D, w.V
    rng = np.random.default_rng([int(seed), int(w.stream)])

    # 1. hidden states
    h = rng.standard_normal((T, D), dtype=np.float32)
    if w.hidden == "unit_rms":
        rms = np.sqrt(np.mean(h.astype(np.float64) ** 2, axis=1, keepdims=True))
        h = (h / rms).astype(np.float32)
    if w.hidden_scale != 1.0:
        h = (h * np.float32(w.hidden_scale)).astype(np.float32)
    # 2. tied embedding
    e = (rng.standard_normal((V, D), dtype=np.float32) * np.float32(w.embed_std)).astype(np.float32)
    # 3. next-token targets
    if w.targets == "uniform":
        y = rng.integers(0, V, size=T, dtype=np.int64)
    elif w.bos_rate is not None:
        y = 1 + _zipf_draw(rng, T, V - 1, w.zipf_s)      # ids 1..V-1; id 0 is kept for BOS
    else:
        y = _zipf_draw(rng, T, V, w.zipf_s)              # id = rank - 1
    # 4. UTF-8 byte length of every vocabulary entry
    if w.bytes_law == "uniform":
        blen = rng.integers(w.bytes_lo, w.bytes_hi + 1, size=V, dtype=np.int64)
    else:
        blen = w.bytes_lo + np.minimum(rng.poisson(w.poisson_lam, size=V), w.bytes_hi - w.bytes_lo)
    # 5. mask and BOS positions
    mask = None
    if w.stride is not None:
        mask = stride_mask(T, w.seq_len, w.stride)
    if w.bos_rate is not None:
        gaps = rng.geometric(w.bos_rate, size=max(16, int(3 * T * w.bos_rate) + 16))
        pos = np.cumsum(gaps) - 1
        y[pos[pos < T]] = 0
        blen[0] = 0

    if w.dtype == "bf16":
        hidden, embed = bf16_bits(h), bf16_bits(e)
    else:
        hidden, embed = h, e
    return dict(
        workload=w.name, seed=int(seed), T=T, D=D, V=V, dtype=w.dtype, softcap=float(w.softcap),
        hidden=np.ascontiguousarray(hidden), embed=np.ascontiguousarray(embed),
        target=y.astype(np.int32), byte_len=blen.astype(np.int32), mask=mask,
    )


def make_stream(seed: int, n_tokens: int, V: int, bos_rate: float = 1.0 / 700.0, D: int = 512,
                embed_std: float = 0.02) -> dict:
    """A token stream for the sliding-window evaluation, drawn from
    ``numpy.random.default_rng([seed, 8])`` in the order embedding, tokens, byte lengths, BOS: a bf16
    N(0, embed_std^2) tied embedding [V, D], Zipf(1.1) token ids over 1..V-1 with BOS (id 0, zero
    bytes) at geometric gaps of mean 1 / bos_rate, and byte lengths 1 + min(Poisson(2.7), 15)."""
    rng = np.random.default_rng([int(seed), 8])
    e = (rng.standard_normal((V, D), dtype=np.float32) * np.float32(embed_std)).astype(np.float32)
    toks = 1 + _zipf_draw(rng, n_tokens, V - 1, 1.1)
    blen = 1 + np.minimum(rng.poisson(2.7, size=V), 15)
    gaps = rng.geometric(bos_rate, size=max(16, int(3 * n_tokens * bos_rate) + 16))
    pos = np.cumsum(gaps) - 1
    toks[pos[pos < n_tokens]] = 0
    blen[0] = 0
    return dict(tokens=toks.astype(np.int32), byte_len=blen.astype(np.int32), embed=bf16_bits(e), V=V, D=D)


def window_hidden(seed: int, w: int, n: int, D: int) -> np.ndarray:
    """Stand-in for the model's hidden states of the n predictions that window w scores (bf16 bits
    [n, D]): unit-RMS rows drawn from ``numpy.random.default_rng([seed, 9, w])``. A position's row
    depends on the window, as a model's does on the window's context."""
    rng = np.random.default_rng([int(seed), 9, int(w)])
    h = rng.standard_normal((n, D), dtype=np.float32)
    rms = np.sqrt(np.mean(h.astype(np.float64) ** 2, axis=1, keepdims=True))
    return bf16_bits((h / rms).astype(np.float32))
