"""Host pieces of the seeded input generator (CPU only)."""
import math

import numpy as np
import pytest


@pytest.fixture(scope="module")
def synth():
    import synth

    return synth


def test_philox_known_answers(synth):
    """Known-answer vectors published with Philox4x32-10 (Random123)."""
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]).tolist() == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2).tolist() == [
        0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]).tolist() \
        == [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_rank_prior(synth):
    rank, base = synth.rank_base(32000, 0)
    assert sorted(rank.tolist()) == list(range(32000))
    assert np.allclose(base, (-0.5 * np.log1p(rank.astype(np.float64))).astype(np.float32), rtol=0, atol=0)
    rank2, _ = synth.rank_base(32000, 1)
    assert (rank != rank2).any()


def test_pacer_scores(synth):
    """The pre-verifier stand-in: U(0,1) scores, reproducible, one Philox block
    per 4 scores of a block (counter (step, b, block, k / 4), stream 6), so a
    sequence's scores do not depend on the batch size."""
    a = synth.pacer_scores(256, 4, 7)
    b = synth.pacer_scores(256, 4, 7)
    assert a.shape == (256, 16) and a.dtype == np.float32 and (a == b).all()
    assert (a >= 0).all() and (a < 1).all() and abs(float(a.mean()) - 0.5) < 0.02
    assert (synth.pacer_scores(3, 4, 7) == a[:3]).all()
    assert not (synth.pacer_scores(256, 4, 8) == a).all()
    ctr = np.array([7, 5, 2, 0], np.uint32)
    key = np.array([4, 6], np.uint32)
    out = np.asarray(synth.philox4x32_10(ctr, key), np.uint32)
    assert np.allclose(a[5, 8:12], (out >> 8).astype(np.float64) / 2 ** 24)


def test_config_table(synth):
    c = synth.CONFIGS
    assert [x.kind for x in c] == ["sd", "sd", "smc", "smc", "sd_ragged", "tree"]
    assert synth.full_tree_parents(2, 3) == [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6]
    assert synth.step_bytes(c[5]) == 64 * (15 + 7) * 32768 * 2 and synth.verified_positions(c[5]) == 64 * 14
    assert synth.step_bytes(c[1]) == 37748736 and synth.verified_positions(c[1]) == 256
    assert synth.step_bytes(c[2]) == 36937728 and c[2].L == 256
    assert synth.step_bytes(c[3]) == 10579607552 and c[3].L == 512
    assert synth.step_bytes(c[0]) == 640000
