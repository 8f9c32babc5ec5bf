"""Local (sliding-chunk) attention on the GPU against the float64 oracle."""
import numpy as np
import pytest

import oracle
from efficient_long_sequence_lsh_amd import workloads as W
from gpu_util import TOL, ensure_library, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nat():
    return ensure_library()


def _say(msg):
    print(msg, flush=True)


def _inputs(B, H, L, d, dtype, seed):
    g = np.random.default_rng(seed)
    arrs = [g.standard_normal((B, H, L, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        bits = [W.f32_to_bf16_bits(a) for a in arrs]
        return [W.bf16_bits_to_f32(b) for b in bits], bits
    return arrs, None


def _device(arrs, bits):
    import torch

    if bits is None:
        return [torch.from_numpy(a).cuda() for a in arrs]
    return [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for b in bits]


@pytest.mark.parametrize("L,d,m,nb,na,causal,dtype", [
    (1024, 64, 64, 1, 0, True, "bf16"),      # the language-model setting: one chunk of look-back
    (1024, 128, 64, 1, 1, False, "f32"),
    (1000, 64, 40, 2, 1, True, "f32"),       # chunks not aligned to key tiles, ragged query tile
    (960, 128, 96, 1, 2, False, "bf16"),
    (256, 64, 1, 0, 0, False, "bf16"),       # windows of one position: out = v
    (320, 128, 320, 0, 0, True, "bf16"),     # one chunk: full causal attention
    (777, 64, 1000, 3, 3, False, "f32"),     # chunk_len > L
    (2048, 64, 128, 1, 1, True, "bf16"),
    (2048, 128, 64, 1, 0, True, "bf16"),     # the 64K text setting's windows: two-slot key ring, two runs
    (2112, 128, 64, 1, 1, False, "bf16"),    # three-slot ring at d = 128, a one-tile last run
    (1280, 64, 64, 1, 0, True, "f32"),       # two-slot ring, float32
    (1536, 128, 64, 1, 0, True, "f32"),      # two-slot ring, float32 at d = 128 (one workgroup per CU)
    (2000, 64, 40, 1, 0, True, "bf16"),      # ring with chunks across tile edges, ragged last tile
    (1280, 64, 64, 0, 1, False, "bf16"),     # two-slot ring, windows reaching ahead (tile counts not regular)
    (1520, 128, 40, 1, 0, True, "bf16"),     # two tiles in flight, three slots, d = 128, ragged last tile
])
def test_local_attention_matches_oracle(nat, L, d, m, nb, na, causal, dtype):
    _say(f"[local] L{L} d{d} m{m} before{nb} after{na} causal={causal} {dtype}")
    (q, k, v), bits = _inputs(2, 2, L, d, dtype, seed=L + m + 3 * nb + na)
    qd, kd, vd = _device([q, k, v], None if bits is None else bits)
    out = host(nat.local_attention(qd, kd, vd, m, nb, na, causal))
    want = oracle.local_attention(q, k, v, m, nb, na, causal)
    err = float(np.abs(out - want).max())
    _say(f"  max abs err {err:.3e}")
    np.testing.assert_allclose(out, want, rtol=0, atol=TOL[dtype])


def test_local_attention_shared_qk(nat):
    """q and k may be the same buffer (no self-mask in local attention)."""
    (q, _, v), bits = _inputs(1, 2, 512, 64, "f32", seed=9)
    import torch

    qd = torch.from_numpy(q).cuda()
    vd = torch.from_numpy(v).cuda()
    out = host(nat.local_attention(qd, qd, vd, 64, 1, 0, True))
    want = oracle.local_attention(q, q, v, 64, 1, 0, True)
    np.testing.assert_allclose(out, want, rtol=0, atol=TOL["f32"])


def test_local_attention_overlaps_beyond_the_sequence(nat):
    """n_before / n_after larger than the number of chunks act as 'all chunks'."""
    (q, k, v), _ = _inputs(1, 1, 256, 64, "f32", seed=4)
    import torch

    qd, kd, vd = (torch.from_numpy(a).cuda() for a in (q, k, v))
    big = host(nat.local_attention(qd, kd, vd, 32, 1 << 30, 1 << 30, False))
    want = oracle.local_attention(q, k, v, 32, 8, 8, False)
    np.testing.assert_allclose(big, want, rtol=0, atol=TOL["f32"])


def test_local_attention_full_size(nat):
    """The 64K text shape in the launch configuration the benchmark times
    (batch 1, 8 heads, L = 65536, d = 128, chunks of 64 with one chunk of
    look-back, causal, bf16): the first and last heads, every row."""
    import torch

    B, H, L, d = 1, 8, 65536, 128
    _say(f"[local-full] B{B} H{H} L{L} d{d}")
    g = np.random.default_rng(20200104)
    bits = [W.f32_to_bf16_bits(g.standard_normal((B, H, L, d), dtype=np.float32)) for _ in range(3)]
    q, k, v = _device(None, bits)
    out = nat.local_attention(q, k, v, 64, 1, 0, True)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        qh, kh, vh = (W.bf16_bits_to_f32(b[0, h]).astype(np.float64) for b in bits)
        want = oracle.local_attention_head(qh, kh, vh, 64, 1, 0, True)
        err = float(np.abs(host(out[0, h]) - want).max())
        _say(f"  head {h}: max abs err {err:.3e}")
        assert err <= TOL["bf16"]
