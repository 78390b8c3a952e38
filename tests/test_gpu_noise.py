"""Device noise against the oracle: Philox words bit-exact, Gumbel variates
within 1e-5 * max(1, |g|) over every one of the 2^23 possible uniforms."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mds():
    import markov_draft_sampling_amd as m
    return m


@pytest.mark.parametrize("seed,pos,salt", [(0, 0, 1 << 30), (-1, (1 << 40) + 5, 1), (123456789012345, 99, 2)])
def test_noise_words_match_oracle(mds, seed, pos, salt):
    import torch
    cols = np.concatenate([np.arange(4096), np.random.default_rng(0).integers(0, 1 << 24, 4096)]).astype(np.int32)
    words, g = mds.debug_noise(torch.from_numpy(cols).cuda(), seed, pos, salt)
    torch.cuda.synchronize()
    want = oracle.noise_words(seed, pos, salt, cols)
    assert np.array_equal(words.cpu().numpy().view(np.uint32), want)
    ref = oracle.gumbel(oracle.uniform24(want))
    err = np.abs(g.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * np.maximum(1.0, np.abs(ref)))


def test_gumbel_exhaustive_over_all_uniforms(mds):
    import torch
    m = np.arange(1 << 23, dtype=np.uint32)
    words = (m << np.uint32(9)) | np.uint32(0x1FF)  # low bits must not matter
    g = mds.debug_gumbel(torch.from_numpy(words.view(np.int32)).cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gumbel(oracle.uniform24(words))
    err = np.abs(g - ref) / np.maximum(1.0, np.abs(ref))
    worst = int(np.argmax(err))
    print(f"max scaled error {err[worst]:.3e} at u={oracle.uniform24(words[worst:worst+1])[0]!r}")
    assert err.max() <= 1e-5
    # endpoints
    assert abs(g[-1] - 16.6355323) < 1e-4 and abs(g[0] - ref[0]) < 1e-5
