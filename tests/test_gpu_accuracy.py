"""More hash rounds bring LSH attention closer to full attention ("Reformer:
The Efficient Transformer" (research summary), Key points, "Number of hash
rounds" bullet).  Full shared-QK attention is this library's pipeline with one
bucket and one chunk spanning the sequence; it is itself checked against the
float64 oracle here, on every head of the shape the accuracy sweep of the
benchmark uses (batch 2, 4 heads, L = 4096, d = 64, causal, float32)."""
import dataclasses

import numpy as np
import pytest

import oracle
from efficient_long_sequence_lsh_amd import workloads as W
from gpu_util import ensure_library, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nat():
    return ensure_library()


@pytest.mark.parametrize("kind,qk_scale", [("normal", 1.0), ("mixture", 1.0), ("mixture", 3.0), ("ar1", 1.0)])
def test_full_attention_reference_matches_oracle_at_sweep_shape(nat, kind, qk_scale):
    import torch

    base = dataclasses.replace(W.WORKLOADS["small_4k_f32"], qk_kind=kind, name=f"sweep_{kind}")
    ref_in = W.make_inputs(dataclasses.replace(base, n_buckets=1, n_rounds=1))
    x = (ref_in.qk * np.float32(qk_scale)).astype(np.float32)
    full = host(nat.attention(torch.from_numpy(x).cuda(), torch.from_numpy(ref_in.v).cuda(), None, 1, base.seq_len,
                              base.causal, n_rounds=1)).astype(np.float64)
    err = 0.0
    for b in range(base.batch):
        for h in range(base.heads):
            want = oracle.lsh_attention_head(x[b, h].astype(np.float64), ref_in.v[b, h].astype(np.float64), None, 1,
                                             base.seq_len, base.causal)["out"]
            err = max(err, float(np.abs(full[b, h] - want).max()))
    print(f"[full-ref] {kind} x{qk_scale}: max abs err {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("kind", ["normal", "mixture", "ar1"])
def test_error_against_full_attention_falls_with_rounds(nat, kind):
    import torch

    base = dataclasses.replace(W.WORKLOADS["small_4k_f32"], batch=1, heads=2, seq_len=2048, qk_kind=kind,
                               name=f"rounds_{kind}")
    ref_in = W.make_inputs(dataclasses.replace(base, n_buckets=1, n_rounds=1))
    qk = torch.from_numpy(ref_in.qk).cuda()
    v = torch.from_numpy(ref_in.v).cuda()
    full = host(nat.attention(qk, v, None, 1, base.seq_len, True, n_rounds=1)).astype(np.float64)
    errs = []
    for r in (1, 2, 4, 8):
        inp = W.make_inputs(dataclasses.replace(base, n_buckets=16, n_rounds=r))
        rot = torch.from_numpy(inp.rotations).cuda()
        out = host(nat.attention(qk, v, rot, 16, 64, True, n_rounds=r)).astype(np.float64)
        errs.append(float(np.linalg.norm(out - full) / np.linalg.norm(full)))
    print(f"[rounds] {kind}: " + " ".join(f"{e:.4f}" for e in errs), flush=True)
    assert errs[-1] < 0.8 * errs[0]
    assert all(b <= 1.02 * a for a, b in zip(errs, errs[1:]))
