"""Seeded synthetic workloads for LSH attention (inputs only).

This module only draws random inputs; it holds none of the attention method's
arithmetic, so both the HIP library's tests and the CPU oracle can consume its
arrays.  Shapes and value distributions follow the workloads the pages name:
the Reformer paper's 64K-token text and 12K-token (64x64x3) image-generation
sequences ("Reformer: The Efficient Transformer", *Summary*) and the
half-million-token sequences of "The Reformer - Pushing the limits of language
modeling", *Summary*.  No dataset is used; the synthetic inputs stand in for
enwik8 / imagenet-64 by shape and structure only.

Generator: ``numpy.random.Generator(PCG64(SeedSequence([20200104, k, s])))``
with ``k`` the workload index and ``s`` the stream (0 = qk, 1 = v,
2 = rotations, 3 = mixture centres and assignments).  Values are drawn in
float64, cast to float32 and, for bf16 workloads, rounded to bfloat16 with
round-to-nearest-even.  The same bytes go to the GPU and to the oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED = 20200104


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    heads: int
    seq_len: int
    d_head: int
    n_buckets: int
    chunk_len: int
    n_rounds: int
    causal: bool
    dtype: str          # "f32" or "bf16"
    qk_kind: str        # "normal", "mixture", "ar1"

    @property
    def head_tokens(self) -> int:
        return self.batch * self.heads * self.seq_len

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def describe(self) -> dict:
        return dataclasses.asdict(self)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_1k", 0, 1, 1, 1024, 64, 32, 32, 1, False, "f32", "normal"),
        Workload("tiny_1k_full", 0, 1, 1, 1024, 64, 1, 1024, 1, False, "f32", "normal"),
        Workload("small_4k_f32", 1, 2, 4, 4096, 64, 64, 64, 2, True, "f32", "normal"),
        Workload("small_4k_bf16", 1, 2, 4, 4096, 64, 64, 64, 2, True, "bf16", "normal"),
        Workload("text_64k", 2, 1, 8, 65536, 128, 1024, 64, 4, True, "bf16", "mixture"),
        Workload("image_12k", 3, 8, 8, 12288, 64, 192, 64, 8, True, "bf16", "ar1"),
        Workload("half_million", 4, 1, 2, 524288, 64, 8192, 64, 8, True, "bf16", "normal"),
    ]
}


def rng(index: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, index, stream])))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Host-side inputs of one workload.

    ``qk`` and ``v`` hold the exact values in float32 (for bf16 workloads these
    are bfloat16 values widened exactly); ``qk_bits`` / ``v_bits`` hold the raw
    bfloat16 bits (uint16) for bf16 workloads and are ``None`` otherwise.
    ``rotations`` is float32 ``[n_rounds, d_head, n_buckets/2]`` (empty second
    axis when ``n_buckets == 1``).
    """

    workload: Workload
    qk: np.ndarray
    v: np.ndarray
    rotations: np.ndarray
    qk_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def _normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float64)


def _mixture_qk(w: Workload) -> np.ndarray:
    """256 centres of norm 3 per head, isotropic noise of expected norm 1."""
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    gc = rng(w.index, 3)
    g = _normal(gc, (B, H, 256, d))
    centres = 3.0 * g / np.linalg.norm(g, axis=-1, keepdims=True)
    assign = gc.integers(0, 256, size=(B, H, L))
    noise = _normal(rng(w.index, 0), (B, H, L, d)) / np.sqrt(d)
    bidx = np.arange(B)[:, None, None]
    hidx = np.arange(H)[None, :, None]
    return centres[bidx, hidx, assign] + noise


def _ar1_qk(w: Workload, rho: float = 0.9) -> np.ndarray:
    """x_0 = e_0, x_t = rho x_{t-1} + e_t with unit-variance normal innovations."""
    from scipy.signal import lfilter

    e = _normal(rng(w.index, 0), (w.batch, w.heads, w.seq_len, w.d_head))
    return lfilter([1.0], [1.0, -rho], e, axis=2)


def make_inputs(w: Workload | str, seq_len: int | None = None) -> Inputs:
    """Draw the inputs of a workload (optionally truncated in length for tests).

    ``seq_len`` replaces the workload's length (the same streams are used, so a
    shorter draw is not a prefix of the full one; it is its own seeded input).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if seq_len is not None:
        w = dataclasses.replace(w, seq_len=int(seq_len))
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    if w.qk_kind == "normal":
        qk = _normal(rng(w.index, 0), (B, H, L, d))
    elif w.qk_kind == "mixture":
        qk = _mixture_qk(w)
    elif w.qk_kind == "ar1":
        qk = _ar1_qk(w)
    else:
        raise ValueError(w.qk_kind)
    v = _normal(rng(w.index, 1), (B, H, L, d))
    half = w.n_buckets // 2 if w.n_buckets > 1 else 0
    rot = _normal(rng(w.index, 2), (w.n_rounds, d, half)).astype(np.float32)
    qk32 = qk.astype(np.float32)
    v32 = v.astype(np.float32)
    if w.dtype == "bf16":
        qb, vb = f32_to_bf16_bits(qk32), f32_to_bf16_bits(v32)
        return Inputs(w, bf16_bits_to_f32(qb), bf16_bits_to_f32(vb), rot, qb, vb)
    if w.dtype != "f32":
        raise ValueError(w.dtype)
    return Inputs(w, qk32, v32, rot)


def custom_inputs(batch, heads, seq_len, d_head, n_buckets, n_rounds, dtype="f32", seed=0, qk_scale=1.0):
    """Small seeded iid-normal inputs of an arbitrary shape (tests and edge cases)."""
    w = Workload(f"custom_{seed}", 100 + seed, batch, heads, seq_len, d_head, n_buckets,
                 max(1, seq_len), n_rounds, False, dtype, "normal")
    g0, g1, g2 = rng(w.index, 0), rng(w.index, 1), rng(w.index, 2)
    qk = (qk_scale * _normal(g0, (batch, heads, seq_len, d_head))).astype(np.float32)
    v = _normal(g1, (batch, heads, seq_len, d_head)).astype(np.float32)
    half = n_buckets // 2 if n_buckets > 1 else 0
    rot = _normal(g2, (n_rounds, d_head, half)).astype(np.float32)
    if dtype == "bf16":
        qb, vb = f32_to_bf16_bits(qk), f32_to_bf16_bits(v)
        return Inputs(w, bf16_bits_to_f32(qb), bf16_bits_to_f32(vb), rot, qb, vb)
    return Inputs(w, qk, v, rot)


def dense_score_matrix_bytes(seq_len: int, batch: int = 1, heads: int = 1, bytes_per_value: int = 4) -> int:
    """Bytes of the full L x L score matrix that chunked LSH attention never builds.

    "Reformer: The Efficient Transformer", *Key points*, memory bullet: at
    64K tokens this matrix is about 16 GB in 32-bit floats at batch size 1.
    """
    return int(batch) * int(heads) * int(seq_len) * int(seq_len) * int(bytes_per_value)
