"""Oracle for the capped (lossy) codebook (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may use this
module; the HIP library and its Python binding never import it.

What it follows.  The codebook overview (how-to section) sets ``codebook_size=8192`` when a model
is compressed, and the Codebook-Quantization digest mentions lossy, "balanced" variants that were
tested less.  With at most K entries a tensor with more than K distinct patterns cannot be stored
exactly; the plainest reading, and the one fixed here, is:

* a tensor with U <= K distinct patterns is left unchanged (the lossless format);
* otherwise K patterns are retained: every Inf/NaN pattern present (exponent field 255), then
  the most frequent of the others, ties broken by the smaller pattern value;
* every other pattern is replaced by the retained finite value nearest to it as a real number,
  ties going to the value closer to zero, then to the smaller pattern;
* the result is then encoded exactly like any tensor (so b <= ceil(log2 K)).

K-means on the values (the digest's AI summary) is the other reading; it was not taken, because
its result depends on initialisation and iteration count, which the pages do not give.

Pinned in ``tests/test_oracle_capped.py`` (hand-worked example, brute-force nearest search on
small inputs, identity when U <= K, invariants).
"""
from __future__ import annotations

import numpy as np


def bf16_to_float(p):
    p = np.asarray(p, dtype=np.uint32)
    return (p << 16).view(np.float32).astype(np.float64)


def is_special(p):
    return ((np.asarray(p, dtype=np.uint32) >> 7) & 0xFF) == 0xFF


def retained_patterns(w, K: int):
    """Sorted (ascending pattern) array of the retained patterns."""
    vals, counts = np.unique(np.asarray(w, dtype=np.uint16).reshape(-1), return_counts=True)
    if vals.size <= K:
        return vals
    spec = is_special(vals)
    if spec.sum() > K or (spec.sum() == K and (~spec).any()):
        raise ValueError("the cap cannot hold the special values and one finite value")
    keep = list(vals[spec])
    others = [(-int(c), int(v)) for v, c in zip(vals[~spec], counts[~spec])]
    others.sort()
    keep += [v for _, v in others[:K - len(keep)]]
    return np.array(sorted(keep), dtype=np.uint16)


def nearest(p: int, finite_retained) -> int:
    """The retained finite pattern nearest to pattern p (ties: closer to zero, then smaller
    pattern), by a scan over all of them."""
    f = float(bf16_to_float(p))
    best = None
    for r in finite_retained:
        fr = float(bf16_to_float(r))
        key = (abs(f - fr), abs(fr), int(r))
        if best is None or key < best[0]:
            best = (key, int(r))
    return best[1]


def cap(w, K: int):
    """The capped tensor: every pattern mapped to itself (retained) or its nearest retained value."""
    w = np.asarray(w, dtype=np.uint16)
    keep = retained_patterns(w, K)
    vals = np.unique(w.reshape(-1))
    if vals.size <= K:
        return w.copy()
    kset = set(int(v) for v in keep)
    fin = np.array([v for v in keep if not is_special(v)], dtype=np.uint16)
    # sort the finite retained values by (value, pattern) for a bisection
    fv = bf16_to_float(fin)
    order = np.lexsort((fin, fv))
    fin, fv = fin[order], fv[order]
    mapping = {}
    for v in vals:
        v = int(v)
        if v in kset:
            mapping[v] = v
            continue
        f = float(bf16_to_float(v))
        i = int(np.searchsorted(fv, f))
        cands = set()
        for j in (i - 2, i - 1, i, i + 1):
            if 0 <= j < fin.size:
                cands.add(int(fin[j]))
        best = min(cands, key=lambda r: (abs(f - float(bf16_to_float(r))), abs(float(bf16_to_float(r))), r))
        mapping[v] = best
    lut = np.zeros(65536, dtype=np.uint16)
    for a, b in mapping.items():
        lut[a] = b
    return lut[w]


def error_metrics(w, wc):
    """Max |error|, RMS error relative to RMS of w, and the fraction of weights changed (finite
    weights only)."""
    a = bf16_to_float(np.asarray(w).reshape(-1))
    b = bf16_to_float(np.asarray(wc).reshape(-1))
    fin = np.isfinite(a)
    d = np.abs(a[fin] - b[fin])
    rms = float(np.sqrt(np.mean(a[fin] ** 2))) if fin.any() else 0.0
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "rel_rms": float(np.sqrt(np.mean(d ** 2)) / rms) if rms > 0 else 0.0,
        "changed": float(np.mean(np.asarray(w).reshape(-1) != np.asarray(wc).reshape(-1))),
    }
