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


def _irwin_hall_cdf(x, n):
    return sum((-1) ** k * math.comb(n, k) * (x - k) ** n for k in range(int(math.floor(x)) + 1)) / math.factorial(n)


def test_pacer_length_law(synth):
    """Blockwise lengths: stop after block m when mean(4 scores) < t, t = 0.5 * 1.1^(m-1)."""
    stop = [_irwin_hall_cdf(4 * 0.5 * 1.1 ** (m - 1), 4) for m in range(1, 4)]
    p = [stop[0], (1 - stop[0]) * stop[1], (1 - stop[0]) * (1 - stop[1]) * stop[2],
         (1 - stop[0]) * (1 - stop[1]) * (1 - stop[2])]
    assert abs(p[1] - 0.31543) < 1e-4 and abs(p[2] - 0.14012) < 1e-4 and abs(p[3] - 0.04444) < 1e-4
    lens = np.concatenate([synth.pacer_lengths(256, 4, s) for s in range(400)])
    assert set(np.unique(lens).tolist()) <= {4, 8, 12, 16}
    n = lens.size
    for m in range(4):
        f = np.mean(lens == 4 * (m + 1))
        assert abs(f - p[m]) < 5 * math.sqrt(p[m] * (1 - p[m]) / n), (m, f, p[m])
    assert abs(lens.mean() - 4 * sum((m + 1) * p[m] for m in range(4))) < 0.05


def test_config_table(synth):
    c = synth.CONFIGS
    assert [x.kind for x in c] == ["sd", "sd", "smc", "smc", "sd_ragged"]
    assert synth.step_bytes(c[1]) == 37748736 and synth.verified_positions(c[1]) == 256
    assert synth.step_bytes(c[2]) == 36937728 and c[2].L == 256
    assert synth.step_bytes(c[3]) == 10579607552 and c[3].L == 512
    assert synth.step_bytes(c[0]) == 640000
