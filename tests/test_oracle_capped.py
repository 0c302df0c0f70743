"""Pins for the capped codebook oracle (oracle/capped.py): a hand-worked example
(tests/golden/capped_worked_example.json), brute-force nearest search on small inputs, identity
when the tensor already fits, and invariants of the rule (size cap, retained values unchanged,
every replaced value no farther than any retained one)."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import capped

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capped_worked_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    w = np.array([int(v, 16) for v in g["w"]], dtype=np.uint16)
    assert capped.retained_patterns(w, g["K"]).tolist() == sorted(int(v, 16) for v in g["retained"])
    assert capped.cap(w, g["K"]).tolist() == [int(v, 16) for v in g["capped"]]


@pytest.mark.parametrize("K", [1, 2, 7, 100])
def test_identity_when_the_tensor_fits(K):
    rng = np.random.default_rng(K)
    w = rng.choice(np.arange(0x3F00, 0x3F00 + K, dtype=np.uint16), 500)
    assert np.array_equal(capped.cap(w, K), w)


@pytest.mark.parametrize("seed", range(6))
def test_invariants_and_brute_force_nearest(seed):
    rng = np.random.default_rng(seed)
    w = synth.gaussian_bf16((3000,), 0.02, seed=[60, seed])
    if seed % 2:
        w[rng.choice(w.size, 5, replace=False)] = np.array([0x7F80, 0xFF80, 0x7FC0, 0x7FC0, 0xFFC1], dtype=np.uint16)
    K = int(rng.integers(8, 300))
    wc = capped.cap(w, K)
    keep = capped.retained_patterns(w, K)
    assert np.unique(wc).size <= K
    assert set(np.unique(wc).tolist()) <= set(keep.tolist())
    # retained patterns and every special value are unchanged
    kept = np.isin(w, keep)
    assert np.array_equal(wc[kept], w[kept])
    assert kept[capped.is_special(w)].all()
    # every replaced pattern went to the nearest retained finite value (scan over all of them)
    fin = [int(v) for v in keep if not capped.is_special(v)]
    for v in np.unique(w[~kept]):
        assert int(wc[np.flatnonzero(w == v)[0]]) == capped.nearest(int(v), fin)
    # retained = most frequent (after the specials): no dropped value is more frequent than a kept
    vals, counts = np.unique(w, return_counts=True)
    cnt = dict(zip(vals.tolist(), counts.tolist()))
    kept_f = [cnt[v] for v in keep.tolist() if not capped.is_special(v)]
    dropped = [cnt[v] for v in vals.tolist() if v not in set(keep.tolist())]
    assert not dropped or max(dropped) <= min(kept_f)


def test_cap_at_8192_keeps_gaussian_tensors_lossless_and_tighter_caps_bound_the_error():
    """A 4096-column N(0, 0.02) tensor has fewer than 8192 distinct patterns (the how-to's
    default cap changes nothing); capping at 2048 (b = 11) changes about 1 % of the weights (the
    rarest patterns: the tails and the tiniest magnitudes) and the RMS error stays under 2 % of
    the RMS weight."""
    w = synth.gaussian_bf16((256, 4096), 0.02, seed=[61])
    assert np.unique(w).size < 8192
    assert np.array_equal(capped.cap(w, 8192), w)
    wc = capped.cap(w, 2048)
    m = capped.error_metrics(w, wc)
    assert np.unique(wc).size <= 2048
    assert 0 < m["changed"] < 0.05
    assert m["rel_rms"] < 0.02


def test_specials_beyond_the_cap_are_rejected():
    w = np.array([0x7F80, 0xFF80, 0x7FC0, 0x3F80], dtype=np.uint16)
    with pytest.raises(ValueError):
        capped.cap(w, 2)
    with pytest.raises(ValueError):
        capped.cap(w, 3)
