"""Gradients of chunk attention + combine on the GPU against the float64
autograd oracle (bucket order held fixed)."""
import numpy as np
import pytest

import oracle
from efficient_long_sequence_lsh_amd import workloads as W
from gpu_util import ensure_library, host, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nat():
    return ensure_library()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("L,d,r,nb,causal,dtype", [
    (256, 64, 1, 8, False, "f32"),
    (512, 64, 2, 16, True, "f32"),
    (512, 128, 3, 8, True, "f32"),
    (1024, 64, 2, 32, True, "bf16"),
    (384, 128, 2, 4, False, "bf16"),
    (64, 64, 2, 4, True, "bf16"),         # one chunk: a single run with no neighbour
    (1600, 128, 2, 16, True, "bf16"),     # 25 chunks: runs of 8, 8, 8 and a last run of one chunk
    (576, 64, 3, 8, False, "bf16"),       # 9 chunks: a full run and a one-chunk run
    (768, 64, 8, 32, True, "bf16"),       # eight rounds (the image-shaped configuration's round count)
])
def test_backward_matches_oracle(nat, L, d, r, nb, causal, dtype):
    import torch

    _say(f"[bwd] L{L} d{d} r{r} b{nb} causal={causal} {dtype}")
    inp = W.custom_inputs(1, 2, L, d, nb, r, dtype=dtype, seed=L + d + r)
    qk, v, rot = to_device(inp)
    b = nat.lsh_hash(qk, rot, nb)
    perm, _ = nat.lsh_sort(b, nb)
    out = nat.attend(qk, v, perm, 64, causal)
    g = np.random.default_rng(L + 1)
    dout_h = g.standard_normal((1, 2, L, d)).astype(np.float32)
    if dtype == "bf16":
        dbits = W.f32_to_bf16_bits(dout_h)
        dout_h = W.bf16_bits_to_f32(dbits)
        dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dout = torch.from_numpy(dout_h).cuda()
    dqk, dv = nat.attend_backward(qk, v, perm, 64, causal, out, dout)
    dqk, dv = host(dqk), host(dv)
    ph = host(perm)
    for h in range(2):
        _, wx, wv = oracle.lsh_attention_head_grad(inp.qk[0, h].astype(np.float64), inp.v[0, h].astype(np.float64),
                                                   ph[0, h], 64, causal, dout_h[0, h].astype(np.float64))
        scale = max(1.0, float(np.abs(wx).max()), float(np.abs(wv).max()))
        tol = (1e-4 if dtype == "f32" else 2e-2) * scale
        ex, ev = float(np.abs(dqk[0, h] - wx).max()), float(np.abs(dv[0, h] - wv).max())
        _say(f"  head {h}: max |dqk err| {ex:.2e}  max |dv err| {ev:.2e}  (scale {scale:.2f})")
        assert ex <= tol and ev <= tol


def _run_length(n_chunks, bh, n_cu=256):
    """The host's choice of chunks per backward workgroup (restated here to
    pick shapes that exercise each run length on a 256-CU part)."""
    best, best_cost = 8, None
    for run in (8, 16, 32):
        wgs = -(-n_chunks // run) * bh
        cost = -(-wgs // n_cu) * (run + 2)
        if best_cost is None or cost < best_cost:
            best, best_cost = run, cost
    return best


@pytest.mark.parametrize("B,H,L,d,r,run", [
    (8, 8, 2560, 64, 2, 16),    # 40 chunks: runs of 16, 16 and 8
    (14, 8, 3840, 64, 2, 32),   # 60 chunks: runs of 32 and 28
])
def test_backward_long_runs(nat, B, H, L, d, r, run):
    """Grids large enough that the backward takes runs of 16 and 32 chunks per
    workgroup (with a shorter last run); heads at both ends of the grid are
    checked against the oracle."""
    import torch

    assert _run_length(L // 64, B * H) == run
    _say(f"[bwd-run] B{B} H{H} L{L} d{d} r{r}: runs of {run}")
    inp = W.custom_inputs(B, H, L, d, 16, r, dtype="bf16", seed=L + B)
    qk, v, rot = to_device(inp)
    b = nat.lsh_hash(qk, rot, 16)
    perm, _ = nat.lsh_sort(b, 16)
    out = nat.attend(qk, v, perm, 64, True)
    g = np.random.default_rng(L + 7)
    dbits = W.f32_to_bf16_bits(g.standard_normal((B, H, L, d)).astype(np.float32))
    dout_h = W.bf16_bits_to_f32(dbits)
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    dqk, dv = nat.attend_backward(qk, v, perm, 64, True, out, dout)
    dqk, dv = host(dqk), host(dv)
    ph = host(perm)
    for bi, h in ((0, 0), (B - 1, H - 1)):
        _, wx, wv = oracle.lsh_attention_head_grad(inp.qk[bi, h].astype(np.float64), inp.v[bi, h].astype(np.float64),
                                                   ph[bi, h], 64, True, dout_h[bi, h].astype(np.float64))
        scale = max(1.0, float(np.abs(wx).max()), float(np.abs(wv).max()))
        ex, ev = float(np.abs(dqk[bi, h] - wx).max()), float(np.abs(dv[bi, h] - wv).max())
        _say(f"  ({bi}, {h}): max |dqk err| {ex:.2e}  max |dv err| {ev:.2e}  (scale {scale:.2f})")
        assert ex <= 2e-2 * scale and ev <= 2e-2 * scale


@pytest.mark.parametrize("name", ["text_64k", "image_12k"])
def test_backward_full_size(nat, name):
    """The backward at the full workload sizes, called as the benchmark times
    it (the forward's log normaliser handed in): gradients at sampled
    positions of the first and last heads against the per-position oracle."""
    import torch

    inp = W.make_inputs(name)
    w = inp.workload
    _say(f"[bwd-full] {name}: B{w.batch} H{w.heads} L{w.seq_len} d{w.d_head} r{w.n_rounds}")
    qk, v, rot = to_device(inp)
    perm, _ = nat.lsh_sort(nat.lsh_hash(qk, rot, w.n_buckets), w.n_buckets)
    out, lse = nat.attend(qk, v, perm, w.chunk_len, w.causal, return_lse=True)
    g = np.random.default_rng(w.index + 17)
    dbits = W.f32_to_bf16_bits(g.standard_normal(tuple(v.shape), dtype=np.float32))
    dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    dqk, dv = nat.attend_backward(qk, v, perm, w.chunk_len, w.causal, out, dout, lse=lse)
    torch.cuda.synchronize()
    L = w.seq_len
    rows = np.unique(np.concatenate([[0, 1, L - 1], g.integers(0, L, size=29)]))
    for bi, h in ((0, 0), (w.batch - 1, w.heads - 1)):
        wx, wv = oracle.grad_positions(inp.qk[bi, h].astype(np.float64), inp.v[bi, h].astype(np.float64),
                                       host(perm[bi, h]), rows, w.chunk_len, w.causal,
                                       W.bf16_bits_to_f32(dbits[bi, h]).astype(np.float64))
        gx, gv = host(dqk[bi, h])[rows], host(dv[bi, h])[rows]
        scale = max(1.0, float(np.abs(wx).max()), float(np.abs(wv).max()))
        ex, ev = float(np.abs(gx - wx).max()), float(np.abs(gv - wv).max())
        _say(f"  ({bi}, {h}): max |dqk err| {ex:.2e}  max |dv err| {ev:.2e}  (scale {scale:.2f})")
        assert ex <= 2e-2 * scale and ev <= 2e-2 * scale


@pytest.mark.parametrize("L,d,r,causal,dtype", [
    (512, 64, 2, True, "f32"),
    (1024, 128, 3, True, "bf16"),
    (640, 64, 4, False, "bf16"),
])
def test_backward_with_forward_normaliser(nat, L, d, r, causal, dtype):
    """attend(..., return_lse=True) gives the combined log normaliser; the
    backward that takes it skips its own normaliser pass and gives the same
    gradients (and the oracle's)."""
    import torch

    _say(f"[bwd-lse] L{L} d{d} r{r} causal={causal} {dtype}")
    nb = 8
    inp = W.custom_inputs(1, 2, L, d, nb, r, dtype=dtype, seed=L + 7 * r)
    qk, v, rot = to_device(inp)
    perm, _ = nat.lsh_sort(nat.lsh_hash(qk, rot, nb), nb)
    out, lse = nat.attend(qk, v, perm, 64, causal, return_lse=True)
    assert torch.equal(out, nat.attend(qk, v, perm, 64, causal))   # the same output with or without lse
    g = np.random.default_rng(L + 3)
    dout_h = g.standard_normal((1, 2, L, d)).astype(np.float32)
    if dtype == "bf16":
        dbits = W.f32_to_bf16_bits(dout_h)
        dout_h = W.bf16_bits_to_f32(dbits)
        dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dout = torch.from_numpy(dout_h).cuda()
    dqk0, dv0 = (host(t) for t in nat.attend_backward(qk, v, perm, 64, causal, out, dout))
    dqk1, dv1 = (host(t) for t in nat.attend_backward(qk, v, perm, 64, causal, out, dout, lse=lse))
    ph = host(perm)
    for h in range(2):
        _, wx, wv = oracle.lsh_attention_head_grad(inp.qk[0, h].astype(np.float64), inp.v[0, h].astype(np.float64),
                                                   ph[0, h], 64, causal, dout_h[0, h].astype(np.float64))
        scale = max(1.0, float(np.abs(wx).max()), float(np.abs(wv).max()))
        tol = (1e-4 if dtype == "f32" else 2e-2) * scale
        e_same = max(float(np.abs(dqk1[0, h] - dqk0[0, h]).max()), float(np.abs(dv1[0, h] - dv0[0, h]).max()))
        ex, ev = float(np.abs(dqk1[0, h] - wx).max()), float(np.abs(dv1[0, h] - wv).max())
        _say(f"  head {h}: lse vs recomputed {e_same:.2e}; vs oracle dqk {ex:.2e} dv {ev:.2e} (scale {scale:.2f})")
        # bf16: P and dS are rounded to bf16 for the gradient contractions, so a
        # normaliser that differs in its last float32 bits can move single
        # roundings by one bf16 step (2^-8 relative)
        assert e_same <= (1e-5 if dtype == "f32" else 4e-3) * scale
        assert ex <= tol and ev <= tol


def test_backward_rejects_other_chunk_lengths(nat):
    import torch

    inp = W.custom_inputs(1, 1, 256, 64, 8, 1, dtype="f32", seed=3)
    qk, v, rot = to_device(inp)
    perm, _ = nat.lsh_sort(nat.lsh_hash(qk, rot, 8), 8)
    out = nat.attend(qk, v, perm, 32, False)
    with pytest.raises(nat.LshError, match="UNSUPPORTED"):
        nat.attend_backward(qk, v, perm, 32, False, out, torch.ones_like(out))
