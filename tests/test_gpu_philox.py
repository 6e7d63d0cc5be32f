"""The device's own random stream, checked directly.

- Philox4x32-10 words against the published known-answer vectors (Salmon et
  al., SC'11, Random123 distribution).
- Philox4x32-10 words against the oracle's separately written Philox on over
  10^6 counters.  These use the counter layout of the verify call (chunk index,
  target row, tag, offset) and edge keys and counters.
- The fp32 Exp(1) noise E = -ln U of every race word, over the whole 2^-24
  grid, against fp64 -ln U: relative error below 4e-7, and +inf at U = 0."""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_05_amd as sv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def device_words(ctr_u32, key):
    c = torch.from_numpy(ctr_u32.view(np.int32)).to(DEV)
    out = sv.spec_verify_debug_philox(c, key)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def test_known_answer_vectors():
    kat = [
        ([0, 0, 0, 0], 0, [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, 0xFFFFFFFFFFFFFFFF, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], 0x299F31D0A4093822,
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        got = device_words(np.array([ctr], np.uint32), key)
        assert got[0].tolist() == want


@pytest.mark.parametrize("key", [0, 1, 0xFFFFFFFFFFFFFFFF, 0x0123456789ABCDEF, 0x9E3779B97F4A7C15])
def test_words_match_the_oracle_on_a_million_counters(key):
    rng = np.random.default_rng(key & 0xFFFF)
    n = 1 << 18
    ctr = np.empty((n, 4), np.uint32)
    # the verify call's layout: (idx >> 2, target row, tag 0..4, offset)
    ctr[:, 0] = rng.integers(0, 1 << 16, n)
    ctr[:, 1] = rng.integers(0, 1 << 20, n)
    ctr[:, 2] = rng.integers(0, 5, n)
    ctr[:, 3] = rng.integers(0, 1 << 32, n, dtype=np.uint64)
    # plus raw counters over the full word range, and edge values
    ctr[: n // 4] = rng.integers(0, 1 << 32, (n // 4, 4), dtype=np.uint64)
    ctr[:8] = [[0, 0, 0, 0], [0xFFFFFFFF] * 4, [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1],
               [0xFFFFFFFF, 0, 0xFFFFFFFF, 0], [0x80000000] * 4]
    got = device_words(ctr, key)
    want = oracle.philox4x32_10_n(ctr, [key & 0xFFFFFFFF, key >> 32])
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    say(f"key {key:#x}: {n} counters, {bad.size} mismatches")
    assert bad.size == 0, f"first mismatch at {ctr[bad[0]]}: {got[bad[0]]} vs {want[bad[0]]}"
    # the oracle's word selection for a few counters of the layout
    for i in range(n // 4, n // 4 + 32):  # counters of the verify layout
        c = ctr[i]
        idx = int(c[0]) * 4 + i % 4
        assert oracle.word(key, int(c[3]), int(c[1]), int(c[2]), idx) == got[i][i % 4]


def test_exp_noise_over_the_whole_grid():
    k = torch.arange(1 << 24, dtype=torch.int64, device=DEV)
    words = ((k << 8) | (k & 0xFF)).to(torch.int32)  # the low 8 bits do not matter
    E = sv.spec_verify_debug_exp_noise(words)
    torch.cuda.synchronize()
    e = E.cpu().numpy().astype(np.float64)
    kk = np.arange(1 << 24, dtype=np.float64)
    assert np.isinf(e[0]) and e[0] > 0
    want = -np.log(kk[1:] * 2.0 ** -24)
    rel = np.abs(e[1:] - want) / want
    worst = int(np.argmax(rel)) + 1
    say(f"exp noise: max relative error {rel.max():.3g} at k = {worst} (U = {worst * 2.0 ** -24:.9g})")
    assert rel.max() < 4e-7
    # spot-check the oracle's noise on the same words
    for kv in [1, 2, 255, 1 << 20, (1 << 23) - 1, 1 << 23, (1 << 24) - 1]:
        assert oracle.uniform_race(kv << 8) == kv * 2.0 ** -24
