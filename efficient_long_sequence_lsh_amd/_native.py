"""ctypes binding over ``libreformer_lsh.so`` (the C ABI in ``include/reformer_lsh.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory (``torch.empty`` on
``cuda``) and the stream (``torch.cuda.current_stream()``).  If the shared
library is missing, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libreformer_lsh.so")

RLSH_F32 = 0
RLSH_BF16 = 1

STATUS = {0: "RLSH_OK", 1: "RLSH_ERR_INVALID_ARGUMENT", 2: "RLSH_ERR_UNSUPPORTED",
          3: "RLSH_ERR_WORKSPACE_TOO_SMALL", 4: "RLSH_ERR_HIP"}

_i = ctypes.c_int
_sz = ctypes.c_size_t
_p = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/reformer_lsh.h
SIGNATURES = {
    "reformer_lsh_status_string": (ctypes.c_char_p, [_i]),
    "reformer_lsh_last_error": (ctypes.c_char_p, []),
    "reformer_lsh_version": (_i, []),
    "reformer_lsh_hash_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "reformer_lsh_hash": (_i, [_p, _i, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "reformer_lsh_hash_noalloc": (_i, [_p, _i, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p]),
    "reformer_lsh_sort_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "reformer_lsh_sort": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "reformer_lsh_chunk_attend": (_i, [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p]),
    "reformer_lsh_combine": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p]),
    "reformer_lsh_attend_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "reformer_lsh_attend": (_i, [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _sz, _p]),
    "reformer_lsh_attend_lse": (_i, [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "reformer_lsh_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "reformer_lsh_attention": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _sz, _p]),
    "reformer_lsh_attention_timed": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _sz, _p, _i, _p]),
    "reformer_lsh_local_attention": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p]),
    "reformer_lsh_attend_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "reformer_lsh_feed_forward_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "reformer_lsh_feed_forward": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _sz, _p]),
    "reformer_lsh_attend_backward": (_i, [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "reformer_lsh_attend_backward_lse": (_i, [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz,
                                              _p]),
}

TIMED_EVENTS = 7   # RLSH_TIMED_EVENTS

_lib = None


class LshError(RuntimeError):
    def __init__(self, name: str, status: int, detail: str):
        super().__init__(f"{name} failed: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m efficient_long_sequence_lsh_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, name: str) -> None:
    if status != 0:
        raise LshError(name, status, lib().reformer_lsh_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RLSH_F32
    if t.dtype == torch.bfloat16:
        return RLSH_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def hash_workspace_bytes(batch, heads, seq_len, d_head, n_rounds, n_buckets) -> int:
    return int(lib().reformer_lsh_hash_workspace_bytes(batch, heads, seq_len, d_head, n_rounds, n_buckets))


def lsh_hash(qk: torch.Tensor, rotations: torch.Tensor | None, n_buckets: int, n_rounds: int | None = None,
             return_near_ties: bool = False):
    """Bucket ids ``int32 [B, H, n_rounds, L]`` of ``qk [B, H, L, d]``."""
    B, H, L, d = qk.shape
    if n_rounds is None:
        if rotations is None:
            raise ValueError("n_rounds is needed when rotations is None")
        n_rounds = rotations.shape[0]
    rot_ptr = None
    if n_buckets > 1:
        if rotations is None or rotations.dtype != torch.float32 or tuple(rotations.shape) != (n_rounds, d, n_buckets // 2):
            raise ValueError("rotations must be float32 [n_rounds, d, n_buckets/2]")
        rot_ptr = _dev(rotations, "rotations")
    buckets = torch.empty((B, H, n_rounds, L), dtype=torch.int32, device=qk.device)
    ties = torch.zeros(1, dtype=torch.int32, device=qk.device)
    nbytes = hash_workspace_bytes(B, H, L, d, n_rounds, n_buckets)
    ws = _ws(nbytes, qk.device)
    st = lib().reformer_lsh_hash(_dev(qk, "qk"), _dtype_code(qk), rot_ptr, B, H, L, d, n_rounds, n_buckets,
                                 buckets.data_ptr(), ties.data_ptr(), ws.data_ptr(), nbytes, _stream())
    _check(st, "reformer_lsh_hash")
    return (buckets, ties) if return_near_ties else buckets


def lsh_hash_noalloc(qk: torch.Tensor, rotations: torch.Tensor | None, n_buckets: int, n_rounds: int | None = None,
                     buckets: torch.Tensor | None = None, near_ties: torch.Tensor | None = None):
    """``reformer_lsh_hash_noalloc``: as ``lsh_hash`` with the library's static
    device scratch instead of a workspace.  ``buckets`` / ``near_ties`` may be
    passed in (then this function allocates nothing either)."""
    B, H, L, d = qk.shape
    if n_rounds is None:
        if rotations is None:
            raise ValueError("n_rounds is needed when rotations is None")
        n_rounds = rotations.shape[0]
    rot_ptr = None
    if n_buckets > 1:
        if rotations is None or rotations.dtype != torch.float32 or tuple(rotations.shape) != (n_rounds, d, n_buckets // 2):
            raise ValueError("rotations must be float32 [n_rounds, d, n_buckets/2]")
        rot_ptr = _dev(rotations, "rotations")
    if buckets is None:
        buckets = torch.empty((B, H, n_rounds, L), dtype=torch.int32, device=qk.device)
    elif buckets.dtype != torch.int32 or tuple(buckets.shape) != (B, H, n_rounds, L):
        raise ValueError("buckets must be int32 [B, H, n_rounds, L]")
    ties_ptr = None if near_ties is None else _dev(near_ties, "near_ties")
    st = lib().reformer_lsh_hash_noalloc(_dev(qk, "qk"), _dtype_code(qk), rot_ptr, B, H, L, d, n_rounds, n_buckets,
                                         _dev(buckets, "buckets"), ties_ptr, _stream())
    _check(st, "reformer_lsh_hash_noalloc")
    return buckets


def sort_workspace_bytes(batch, heads, seq_len, n_rounds, n_buckets) -> int:
    return int(lib().reformer_lsh_sort_workspace_bytes(batch, heads, seq_len, n_rounds, n_buckets))


def lsh_sort(buckets: torch.Tensor, n_buckets: int, inverse: bool = True):
    """Stable sort by bucket: returns ``(perm, inv)`` (``inv`` is None unless ``inverse``)."""
    if buckets.dtype != torch.int32:
        raise TypeError("buckets must be int32")
    B, H, r, L = buckets.shape
    perm = torch.empty_like(buckets)
    inv = torch.empty_like(buckets) if inverse else None
    nbytes = sort_workspace_bytes(B, H, L, r, n_buckets)
    ws = _ws(nbytes, buckets.device)
    st = lib().reformer_lsh_sort(_dev(buckets, "buckets"), B, H, L, r, n_buckets, perm.data_ptr(),
                                 None if inv is None else inv.data_ptr(), ws.data_ptr(), nbytes, _stream())
    _check(st, "reformer_lsh_sort")
    return perm, inv


def _check_pair(qk, v):
    if qk.shape != v.shape or qk.dtype != v.dtype:
        raise ValueError("qk and v must have the same shape and dtype")


def chunk_attend(qk: torch.Tensor, v: torch.Tensor, perm: torch.Tensor, chunk_len: int, causal: bool):
    """Per-round ``(o [B,H,r,L,d] float32, z [B,H,r,L] float32)`` in position order."""
    _check_pair(qk, v)
    B, H, L, d = qk.shape
    r = perm.shape[2]
    if perm.dtype != torch.int32 or tuple(perm.shape) != (B, H, r, L):
        raise ValueError("perm must be int32 [B, H, n_rounds, L]")
    o = torch.empty((B, H, r, L, d), dtype=torch.float32, device=qk.device)
    z = torch.empty((B, H, r, L), dtype=torch.float32, device=qk.device)
    st = lib().reformer_lsh_chunk_attend(_dev(qk, "qk"), _dev(v, "v"), _dtype_code(qk), _dev(perm, "perm"), B, H, L, d,
                                         r, int(chunk_len), int(bool(causal)), o.data_ptr(), z.data_ptr(), _stream())
    _check(st, "reformer_lsh_chunk_attend")
    return o, z


def combine(o_rounds: torch.Tensor, z_rounds: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    B, H, r, L, d = o_rounds.shape
    out = torch.empty_like(v)
    st = lib().reformer_lsh_combine(_dev(o_rounds, "o_rounds"), _dev(z_rounds, "z_rounds"), _dev(v, "v"),
                                    _dtype_code(v), B, H, L, d, r, out.data_ptr(), _stream())
    _check(st, "reformer_lsh_combine")
    return out


def attend(qk: torch.Tensor, v: torch.Tensor, perm: torch.Tensor, chunk_len: int, causal: bool,
           return_lse: bool = False):
    """``out`` (input dtype, ``[B, H, L, d]``); with ``return_lse`` also the
    float32 ``[B, H, L]`` log normaliser (``reformer_lsh_attend_lse``)."""
    _check_pair(qk, v)
    B, H, L, d = qk.shape
    r = perm.shape[2]
    nbytes = int(lib().reformer_lsh_attend_workspace_bytes(_dtype_code(qk), B, H, L, d, r, int(chunk_len)))
    ws = _ws(nbytes, qk.device)
    out = torch.empty_like(v)
    if return_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=qk.device)
        st = lib().reformer_lsh_attend_lse(_dev(qk, "qk"), _dev(v, "v"), _dtype_code(qk), _dev(perm, "perm"), B, H, L,
                                           d, r, int(chunk_len), int(bool(causal)), out.data_ptr(), lse.data_ptr(),
                                           ws.data_ptr(), nbytes, _stream())
        _check(st, "reformer_lsh_attend_lse")
        return out, lse
    st = lib().reformer_lsh_attend(_dev(qk, "qk"), _dev(v, "v"), _dtype_code(qk), _dev(perm, "perm"), B, H, L, d, r,
                                   int(chunk_len), int(bool(causal)), out.data_ptr(), ws.data_ptr(), nbytes, _stream())
    _check(st, "reformer_lsh_attend")
    return out


def workspace_bytes(batch, heads, seq_len, d_head, n_rounds, n_buckets, chunk_len, dtype=RLSH_BF16) -> int:
    """Workspace of reformer_lsh_attention; dtype is RLSH_F32 / RLSH_BF16 (or a torch dtype)."""
    if not isinstance(dtype, int):
        dtype = RLSH_BF16 if dtype == torch.bfloat16 else RLSH_F32
    return int(lib().reformer_lsh_workspace_bytes(dtype, batch, heads, seq_len, d_head, n_rounds, n_buckets,
                                                  chunk_len))


def attention(qk: torch.Tensor, v: torch.Tensor, rotations: torch.Tensor | None, n_buckets: int, chunk_len: int,
              causal: bool, n_rounds: int | None = None, workspace: torch.Tensor | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """Whole forward pass (hash, sort, chunk attention, combine) -> ``out [B, H, L, d]``."""
    _check_pair(qk, v)
    B, H, L, d = qk.shape
    if n_rounds is None:
        if rotations is None:
            raise ValueError("n_rounds is needed when rotations is None")
        n_rounds = rotations.shape[0]
    rot_ptr = None
    if n_buckets > 1:
        if rotations is None or rotations.dtype != torch.float32 or tuple(rotations.shape) != (n_rounds, d, n_buckets // 2):
            raise ValueError("rotations must be float32 [n_rounds, d, n_buckets/2]")
        rot_ptr = _dev(rotations, "rotations")
    nbytes = workspace_bytes(B, H, L, d, n_rounds, n_buckets, chunk_len, _dtype_code(qk))
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = _ws(nbytes, qk.device)
    if out is None:
        out = torch.empty_like(v)
    st = lib().reformer_lsh_attention(_dev(qk, "qk"), _dev(v, "v"), rot_ptr, _dtype_code(qk), B, H, L, d, n_rounds,
                                      n_buckets, int(chunk_len), int(bool(causal)), _dev(out, "out"),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    _check(st, "reformer_lsh_attention")
    return out


def local_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, chunk_len: int, n_before: int, n_after: int,
                    causal: bool, out: torch.Tensor | None = None) -> torch.Tensor:
    """Local (sliding-chunk) attention over separate ``q, k, v [B, H, L, d]`` -> ``out``."""
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k and v must have the same shape and dtype")
    B, H, L, d = q.shape
    if out is None:
        out = torch.empty_like(v)
    st = lib().reformer_lsh_local_attention(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), B, H, L, d,
                                            int(chunk_len), int(n_before), int(n_after), int(bool(causal)),
                                            _dev(out, "out"), _stream())
    _check(st, "reformer_lsh_local_attention")
    return out


def attend_backward(qk: torch.Tensor, v: torch.Tensor, perm: torch.Tensor, chunk_len: int, causal: bool,
                    out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor | None = None):
    """Gradients ``(dqk, dv)`` (float32 ``[B, H, L, d]``) of ``attend`` for a fixed sorted order;
    ``lse`` (the forward's, from ``attend(..., return_lse=True)``) skips the normaliser pass."""
    _check_pair(qk, v)
    _check_pair(out, dout)
    B, H, L, d = qk.shape
    r = perm.shape[2]
    if perm.dtype != torch.int32 or tuple(perm.shape) != (B, H, r, L):
        raise ValueError("perm must be int32 [B, H, n_rounds, L]")
    nbytes = int(lib().reformer_lsh_attend_backward_workspace_bytes(B, H, L, d, r, int(chunk_len)))
    ws = _ws(nbytes, qk.device)
    dqk = torch.empty((B, H, L, d), dtype=torch.float32, device=qk.device)
    dv = torch.empty_like(dqk)
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L):
            raise ValueError("lse must be float32 [B, H, L]")
        st = lib().reformer_lsh_attend_backward_lse(_dev(qk, "qk"), _dev(v, "v"), _dtype_code(qk), _dev(perm, "perm"),
                                                    B, H, L, d, r, int(chunk_len), int(bool(causal)), _dev(out, "out"),
                                                    _dev(dout, "dout"), _dev(lse, "lse"), dqk.data_ptr(),
                                                    dv.data_ptr(), ws.data_ptr(), nbytes, _stream())
        _check(st, "reformer_lsh_attend_backward_lse")
        return dqk, dv
    st = lib().reformer_lsh_attend_backward(_dev(qk, "qk"), _dev(v, "v"), _dtype_code(qk), _dev(perm, "perm"), B, H, L,
                                            d, r, int(chunk_len), int(bool(causal)), _dev(out, "out"),
                                            _dev(dout, "dout"), dqk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nbytes,
                                            _stream())
    _check(st, "reformer_lsh_attend_backward")
    return dqk, dv


def feed_forward(x: torch.Tensor, w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: torch.Tensor,
                 chunk_tokens: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """``relu(x W1^T + b1) W2^T + b2`` over ``x [n, d_model]`` (bf16) in chunks of positions."""
    if x.dtype != torch.bfloat16 or w1.dtype != torch.bfloat16 or w2.dtype != torch.bfloat16:
        raise TypeError("x, w1 and w2 must be bfloat16")
    if b1.dtype != torch.float32 or b2.dtype != torch.float32:
        raise TypeError("b1 and b2 must be float32")
    n, d = x.shape
    f = w1.shape[0]
    if tuple(w1.shape) != (f, d) or tuple(w2.shape) != (d, f) or b1.numel() != f or b2.numel() != d:
        raise ValueError("shapes: x [n, d], w1 [f, d], b1 [f], w2 [d, f], b2 [d]")
    nbytes = int(lib().reformer_lsh_feed_forward_workspace_bytes(n, d, f, int(chunk_tokens)))
    ws = _ws(nbytes, x.device)
    if out is None:
        out = torch.empty_like(x)
    st = lib().reformer_lsh_feed_forward(_dev(x, "x"), _dev(w1, "w1"), _dev(b1, "b1"), _dev(w2, "w2"), _dev(b2, "b2"),
                                         n, d, f, int(chunk_tokens), _dev(out, "out"), ws.data_ptr(), nbytes,
                                         _stream())
    _check(st, "reformer_lsh_feed_forward")
    return out
