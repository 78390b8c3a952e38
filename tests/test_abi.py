"""The C-ABI library loads and exports every entry point include/mds.h
declares, and its host-side validation rejects bad arguments without any
device work (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mds.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mds_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from markov_draft_sampling_amd import build, library_path
    if not os.path.exists(library_path()):
        build.build()
    return ctypes.CDLL(library_path())


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("mds_markov_draft_loop", "mds_rejection_verify", "mds_draft_workspace_bytes",
              "mds_verify_workspace_bytes", "mds_abi_version", "mds_status_string", "mds_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version(lib):
    import markov_draft_sampling_amd as mds
    assert mds.abi_version() == 2


def test_workspace_queries_validate_sizes():
    import markov_draft_sampling_amd as mds
    assert mds.draft_workspace_bytes(32, 7, 200064, 256) > 0
    assert mds.verify_workspace_bytes(32, 7, 200064, True, False) > mds.verify_workspace_bytes(32, 7, 200064, False,
                                                                                               True)
    with pytest.raises(mds.MdsError, match="invalid argument"):
        mds.draft_workspace_bytes(0, 7, 1000, 64)
    with pytest.raises(mds.MdsError, match="invalid argument"):
        mds.draft_workspace_bytes(1, 33, 1000, 64)
    with pytest.raises(mds.MdsError, match="invalid argument"):
        mds.draft_workspace_bytes(1, 3, 1, 64)
    with pytest.raises(mds.MdsError, match="unsupported"):
        mds.draft_workspace_bytes(1, 3, 1000, 72)
    with pytest.raises(mds.MdsError, match="invalid argument"):
        mds.draft_workspace_bytes(1, 3, 1000, 1024)


def test_draft_loop_rejects_bad_arguments_on_the_host(lib):
    # all pointers NULL: rejected before anything reaches the device
    f = lib.mds_markov_draft_loop
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [ctypes.c_int] * 4 + [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64,
                                       vp, vp, vp, ctypes.c_size_t, vp]
    f.restype = ctypes.c_int
    args = [4, 3, 1000, 64] + [None, 0, 3000, 1000] + [None] * 7 + [0, 3000, 1000, None, None, None, 0, None]
    assert f(*args) == -1
    args[:4] = [4, 3, 1000, 48]
    assert f(*args) == -2  # rank not a multiple of 32
    lib.mds_last_error.restype = ctypes.c_char_p
    assert lib.mds_last_error()


def test_verify_rejects_bad_arguments_on_the_host(lib):
    f = lib.mds_rejection_verify
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [ctypes.c_int] * 3 + [vp, i64, vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    f.restype = ctypes.c_int
    fake = 1 << 20  # never dereferenced: validation fails first
    args = [2, 3, 1000, fake, 999, fake, 0, 3000, 1000, None, fake, fake, None, fake, fake, fake, fake, fake, 1 << 30,
            None]
    assert f(*args) == -1  # target row stride < V
    args[4] = 1000
    args[18] = 16  # workspace far too small
    assert f(*args) == -3
    args[6] = 5  # bad dtype
    assert f(*args) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import markov_draft_sampling_amd as mds
    monkeypatch.setattr(mds, "_LIB", None)
    monkeypatch.setattr(mds, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(mds.MdsError, match="missing"):
        mds.abi_version()


def test_verify_counter_block_layout():
    # every request of the largest batch has its own counter and its own key
    # in the fixed block, and no key overlaps any counter
    import numpy as np
    import markov_draft_sampling_amd as mds
    n = 65535
    cnt = np.empty(n, np.int64)
    key = np.empty(n, np.int64)
    for b in range(n):
        cnt[b], key[b] = mds.verify_slot_offsets(b)
    lo, hi = 256, 256 + (1 << 20)
    assert cnt.min() >= lo and cnt.max() + 4 <= hi and key.min() >= lo and key.max() + 8 <= hi
    assert np.all(cnt % 4 == 0) and np.all(key % 8 == 0)
    assert np.unique(cnt).size == n and np.unique(key).size == n
    cover = np.zeros(hi, np.int8)
    for off in range(4):
        cover[cnt + off] += 1
    for off in range(8):
        cover[key + off] += 1
    assert cover.max() == 1  # no byte belongs to two words
    # requests b and b + 2048 i share a 512-byte line; no other two do
    line = (cnt - lo) // 512
    assert np.array_equal(line, (key - lo) // 512)
    assert np.array_equal(line, np.arange(n) % 2048)
    with pytest.raises(mds.MdsError, match="invalid argument"):
        mds.verify_slot_offsets(65535)


def test_tiled_w2_size_and_host_validation():
    import markov_draft_sampling_amd as mds
    # 32 r bytes per 16-row tile, the last tile padded
    assert mds.markov_w2_tiled_bytes(200064, 256) == 12504 * 16 * 256 * 2
    assert mds.markov_w2_tiled_bytes(33001, 256) == 2063 * 16 * 256 * 2
    assert mds.markov_w2_tiled_bytes(17, 512) == 2 * 16 * 512 * 2
    with pytest.raises(mds.MdsError, match="invalid argument"):
        mds.markov_w2_tiled_bytes(1, 256)
    with pytest.raises(mds.MdsError, match="unsupported"):
        mds.markov_w2_tiled_bytes(1000, 48)
    f = mds._lib().mds_tile_markov_w2
    fake, need = 1 << 24, 63 * 16 * 64 * 2  # addresses never dereferenced: validation fails first
    assert f(1000, 64, None, fake, need, None) == -1
    assert f(1000, 64, fake + 8, fake + (1 << 22), need, None) == -1  # misaligned
    assert f(1000, 64, fake, fake + (1 << 22), need - 16, None) == -1  # too short
    assert f(1000, 64, fake, fake + 1000 * 64, need, None) == -1  # overlaps w2


def test_tiled_w2_flag_limits_on_the_host():
    import markov_draft_sampling_amd as mds
    lib = mds._lib()
    fake = 1 << 24
    B, K, V = 2, 3, 1000
    # _ex: tiled w2 with rank 512 is unsupported (checked before any device work)
    args = [B, K, V, 512, fake, mds.F32, K * V, V, fake, fake, fake, None, fake, B, fake, fake, None, B, fake,
            mds.F32, K * V, V, fake, None, mds.DRAFT_W2_TILED, fake, 1 << 30, None, None, None, None]
    assert lib.mds_markov_draft_loop_ex(*args) == -2
    args[24] = 4  # unknown flag bit
    assert lib.mds_markov_draft_loop_ex(*args) == -1
    # top-k drafting reads row-major w2 only
    targs = [B, K, V, 256, 8] + args[4:]
    targs[5 + 24 - 4] = mds.DRAFT_W2_TILED
    targs = targs[:-1]  # no launch-count argument
    assert lib.mds_markov_draft_loop_topk(*targs) == -2
