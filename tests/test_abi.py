"""The C ABI loads, exports every declared symbol, and rejects bad arguments on
the host before any HIP call (no GPU needed)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "reformer_lsh.h")


@pytest.fixture(scope="module")
def lib():
    from efficient_long_sequence_lsh_amd import _native

    if not os.path.exists(_native.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    return _native.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(reformer_lsh_\w+)\s*\(", text)))


def test_header_declares_the_pipeline():
    names = declared_functions()
    for want in ["reformer_lsh_hash", "reformer_lsh_sort", "reformer_lsh_chunk_attend", "reformer_lsh_combine",
                 "reformer_lsh_attend", "reformer_lsh_attention", "reformer_lsh_workspace_bytes",
                 "reformer_lsh_status_string", "reformer_lsh_last_error"]:
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    from efficient_long_sequence_lsh_amd import _native

    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _native.SIGNATURES, f"binding lacks {name}"


def test_status_strings(lib):
    assert lib.reformer_lsh_status_string(0) == b"RLSH_OK"
    assert lib.reformer_lsh_status_string(3) == b"RLSH_ERR_WORKSPACE_TOO_SMALL"
    assert lib.reformer_lsh_version() >= 10000


FAKE = 0x1000  # never dereferenced: validation fails before any HIP call


@pytest.mark.parametrize("args,code", [
    # qk, v, rot, dtype, B, H, L, d, r, nb, m, causal, out, ws, wsb
    ((None, FAKE, FAKE, 1, 1, 1, 128, 64, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 1),        # null qk
    ((FAKE, FAKE, FAKE, 1, 0, 1, 128, 64, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 1),        # batch 0
    ((FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 1, 7, 32, 0, FAKE, FAKE, 1 << 30), 1),        # odd buckets
    ((FAKE, FAKE, FAKE, 1, 1, 1, 100, 64, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 1),        # L % m != 0
    ((FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 1, 8, 0, 0, FAKE, FAKE, 1 << 30), 1),         # chunk 0
    ((FAKE, FAKE, FAKE, 1, 1, 1, 128, 96, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 2),        # d = 96
    ((FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 1, 1 << 15, 32, 0, FAKE, FAKE, 1 << 30), 2),  # too many buckets
    ((FAKE, FAKE, FAKE, 7, 1, 1, 128, 64, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 1),        # bad dtype
    ((FAKE, FAKE, None, 1, 1, 1, 128, 64, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 1),        # no rotations
    ((FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 1, 8, 32, 0, FAKE, FAKE, 16), 3),             # workspace short
    ((FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 1, 8, 32, 0, FAKE, None, 1 << 30), 3),        # no workspace
    ((FAKE, FAKE, FAKE, 1, 1 << 14, 1 << 14, 64, 64, 1, 8, 32, 0, FAKE, FAKE, 1 << 30), 1),  # too large
])
def test_attention_rejects_bad_arguments(lib, args, code):
    st = lib.reformer_lsh_attention(*args, None)
    assert st == code, lib.reformer_lsh_last_error()
    assert lib.reformer_lsh_last_error()


def test_noalloc_hash_rejects_bad_arguments_before_any_hip_call(lib):
    # null buckets
    assert lib.reformer_lsh_hash_noalloc(FAKE, 1, FAKE, 1, 1, 64, 64, 1, 8, None, None, None) == 1
    # no rotations with several buckets
    assert lib.reformer_lsh_hash_noalloc(FAKE, 1, None, 1, 1, 64, 64, 1, 8, FAKE, None, None) == 1
    # scratch beyond the static array (4 heads of 512K positions, 8 rounds, 8192 buckets): rejected by size
    assert lib.reformer_lsh_hash_noalloc(FAKE, 1, FAKE, 1, 4, 524288, 64, 8, 8192, FAKE, None, None) == 2
    assert b"static scratch" in lib.reformer_lsh_last_error()


def test_stage_entry_points_reject_bad_arguments(lib):
    # hash: null buckets
    assert lib.reformer_lsh_hash(FAKE, 1, FAKE, 1, 1, 64, 64, 1, 8, None, None, FAKE, 1 << 20, None) == 1
    # hash: short workspace
    assert lib.reformer_lsh_hash(FAKE, 1, FAKE, 1, 1, 64, 64, 1, 8, FAKE, None, FAKE, 4, None) == 3
    # sort: null perm, bad bucket count
    assert lib.reformer_lsh_sort(FAKE, 1, 1, 64, 1, 8, None, None, FAKE, 1 << 20, None) == 1
    assert lib.reformer_lsh_sort(FAKE, 1, 1, 64, 1, 3, FAKE, None, FAKE, 1 << 20, None) == 1
    # chunk_attend: null o, ragged chunk
    assert lib.reformer_lsh_chunk_attend(FAKE, FAKE, 1, FAKE, 1, 1, 64, 64, 1, 32, 0, None, FAKE, None) == 1
    assert lib.reformer_lsh_chunk_attend(FAKE, FAKE, 1, FAKE, 1, 1, 64, 64, 1, 48, 0, FAKE, FAKE, None) == 1
    # combine: unsupported d
    assert lib.reformer_lsh_combine(FAKE, FAKE, FAKE, 0, 1, 1, 64, 32, 1, FAKE, None) == 2
    # attend: short workspace
    assert lib.reformer_lsh_attend(FAKE, FAKE, 1, FAKE, 1, 1, 64, 64, 1, 32, 0, FAKE, FAKE, 8, None) == 3


def test_workspace_sizes(lib):
    n = 8 * 65536 * 4
    full32 = lib.reformer_lsh_workspace_bytes(0, 1, 8, 65536, 128, 4, 1024, 64)
    assert full32 >= n * 128 * 4 + n * 4 * 3      # float32 o + z + buckets + perm
    assert full32 < n * 128 * 4 * 1.2
    full16 = lib.reformer_lsh_workspace_bytes(1, 1, 8, 65536, 128, 4, 1024, 64)
    # bf16 with 64-slot chunks: compact rounds (192-byte rows of 12-bit values at d = 128, their z in
    # the rows' own bits) + buckets + perm, or the hash scratch where that is larger
    assert n * 192 + n * 8 <= full16 < n * 128 * 2 + n * 8
    # bf16 with other chunk lengths keeps float32 rounds
    assert lib.reformer_lsh_workspace_bytes(1, 1, 8, 65536, 128, 4, 1024, 32) >= n * 128 * 4
    assert lib.reformer_lsh_workspace_bytes(1, 1, 8, 65536, 96, 4, 1024, 64) == 0   # invalid -> 0
    assert lib.reformer_lsh_workspace_bytes(5, 1, 8, 65536, 128, 4, 1024, 64) == 0  # bad dtype -> 0
    assert lib.reformer_lsh_hash_workspace_bytes(1, 1, 1024, 64, 1, 1) == 0       # one bucket: no scratch
    # one workgroup per segment (<= 12288 positions, <= 256 buckets): no scratch
    assert lib.reformer_lsh_sort_workspace_bytes(2, 4, 4096, 2, 64) == 0
    # tiles of 4096: per-tile bin counts and bin totals
    assert lib.reformer_lsh_sort_workspace_bytes(1, 8, 65536, 4, 1024) >= 32 * 16 * 1024 * 4 + 32 * 1024 * 4
    # two passes: 4-byte entries per position and round on top of the counts
    assert lib.reformer_lsh_sort_workspace_bytes(1, 2, 524288, 8, 8192) >= 16 * 524288 * 4
    assert lib.reformer_lsh_attend_workspace_bytes(0, 2, 4, 4096, 64, 2, 64) >= 2 * 4 * 4096 * 2 * 65 * 4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from efficient_long_sequence_lsh_amd import _native

    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _native.lib()


def test_local_attention_rejects_bad_arguments(lib):
    # q, k, v, dtype, B, H, L, d, chunk_len, n_before, n_after, causal, out, stream
    call = lib.reformer_lsh_local_attention
    assert call(FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 32, -1, 0, 0, FAKE, None) == 1      # negative overlap
    assert call(FAKE, FAKE, FAKE, 1, 1, 1, 128, 96, 32, 1, 0, 0, FAKE, None) == 2       # d = 96
    assert call(None, FAKE, FAKE, 1, 1, 1, 128, 64, 32, 1, 0, 0, FAKE, None) == 1       # null q
    assert call(FAKE, FAKE, FAKE, 1, 1, 1, 100, 64, 32, 1, 0, 0, FAKE, None) == 1       # L % chunk
    assert call(FAKE, FAKE, FAKE, 1, 1, 1, 128, 64, 0, 1, 0, 0, FAKE, None) == 1        # chunk 0
    assert call(FAKE + 4, FAKE, FAKE, 1, 1, 1, 128, 64, 32, 1, 0, 0, FAKE, None) == 1   # misaligned q
    assert lib.reformer_lsh_last_error()


def test_feed_forward_rejects_bad_arguments(lib):
    # x, w1, b1, w2, b2, n_tokens, d_model, d_ff, chunk_tokens, out, ws, wsb, stream
    call = lib.reformer_lsh_feed_forward
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 96, 256, 0, FAKE, FAKE, 1 << 30, None) == 2      # d_model 96
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 128, 200, 0, FAKE, FAKE, 1 << 30, None) == 2     # d_ff 200
    assert call(None, FAKE, FAKE, FAKE, FAKE, 100, 128, 256, 0, FAKE, FAKE, 1 << 30, None) == 1     # null x
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 128, 256, 0, FAKE, FAKE, 1 << 30, None) == 1       # no tokens
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 128, 256, -1, FAKE, FAKE, 1 << 30, None) == 1    # chunk < 0
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 128, 256, 0, FAKE, FAKE, 16, None) == 3          # workspace
    assert lib.reformer_lsh_feed_forward_workspace_bytes(1000, 128, 256, 64) == 64 * 256 * 2
    assert lib.reformer_lsh_feed_forward_workspace_bytes(1000, 128, 256, 0) >= 1000 * 256 * 2


def test_normaliser_entry_points_reject_bad_arguments(lib):
    # attend_lse: qk, v, dtype, perm, B, H, L, d, r, m, causal, out, lse, ws, wsb, stream
    call = lib.reformer_lsh_attend_lse
    assert call(FAKE, FAKE, 1, FAKE, 1, 1, 256, 64, 2, 64, 1, FAKE, None, FAKE, 1 << 30, None) == 1       # null lse
    assert call(FAKE, FAKE, 1, FAKE, 1, 1, 256, 96, 2, 64, 1, FAKE, FAKE, FAKE, 1 << 30, None) == 2       # d_head 96
    assert call(FAKE, FAKE, 1, FAKE, 1, 1, 256, 64, 2, 64, 1, FAKE, FAKE, FAKE, 16, None) == 3            # workspace
    # backward_lse: qk, v, dtype, perm, B, H, L, d, r, m, causal, out, dout, lse, dqk, dv, ws, wsb, stream
    call = lib.reformer_lsh_attend_backward_lse
    assert call(FAKE, FAKE, 1, FAKE, 1, 1, 256, 64, 2, 64, 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30,
                None) == 1                                                                                # null lse
    assert call(FAKE, FAKE, 1, FAKE, 1, 1, 256, 64, 2, 32, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                None) == 2                                                                                # 32-slot chunks
    assert call(FAKE, FAKE, 1, FAKE, 1, 1, 256, 64, 2, 64, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                None) == 3                                                                                # workspace
