"""Oracle for the exponent-entropy-coded BF16 format (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may use this
module; the HIP library and its Python binding never import it.

What the format follows.  The DFloat11 article (gadzety360.pl, "Przełom: DFloat11" and "Jak to
działa w praktyce?") describes lossless BF16 compression that keeps the sign and the 7 mantissa
bits as they are and entropy-codes (Huffman) only the 8 exponent bits, because the exponent
carries far less information than its width; the decoder uses small lookup tables held in on-chip
memory and a two-phase kernel in which threads first find how many values they will decode and,
after a synchronisation, write them to their places.  Where the article is silent this module
fixes the plainest reading, and the HIP library implements the same bytes:

* per weight, ``sm = (sign << 7) | mantissa`` is stored as one raw byte; ``e`` (bits 7..14) is coded;
* the code is an optimal prefix code over the exponent values present, with lengths capped at
  ``L_MAX = 12`` bits (optimal among codes with that cap; the package-merge method of Larmore and
  Hirschberg computes one); a tensor with one exponent value gets a 1-bit code;
* codes are canonical: ordered by (length, exponent value), each the previous one plus one,
  shifted left when the length grows;
* the code bits are written first bit first into a little-endian uint32 stream read LSB first
  (so the stored field of a code is its bit-reversal);
* the stream is cut into spans of 64 bits; ``gap[j]`` (4 bits, eight to a uint32) is the offset of
  the first code that starts in span j (the stream end if none starts there), so span j can be
  decoded on its own; spans are grouped 256 to a block and ``base[k]`` is the index of the first
  value whose code starts in block k;
* a 4,096-entry table maps the next 12 stream bits to ``exponent | length << 8`` (entries no code
  reaches hold ``12 << 8``).

Every function is pinned in ``tests/test_oracle_entropy.py``: a hand-worked stream in
``tests/golden/entropy_worked_example.json``, brute force over all length vectors for small
alphabets, a heap-based Huffman cost where the cap does not bind, Kraft equality, a textbook
Huffman example, and round trips through an independent bit-by-bit decoder.
"""
from __future__ import annotations

import heapq
import itertools

import numpy as np

L_MAX = 12
SPAN_BITS = 64
BLOCK_SPANS = 256
LUT_BITS = 12


def split(w):
    """(exponent, sign-mantissa byte) of each 16-bit pattern."""
    w = np.asarray(w, dtype=np.uint16).reshape(-1).astype(np.uint32)
    e = ((w >> 7) & 0xFF).astype(np.uint8)
    sm = (((w >> 8) & 0x80) | (w & 0x7F)).astype(np.uint8)
    return e, sm


def join(e, sm):
    """The 16-bit patterns back from exponents and sign-mantissa bytes."""
    e = np.asarray(e, dtype=np.uint32)
    sm = np.asarray(sm, dtype=np.uint32)
    return (((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F)).astype(np.uint16)


def optimal_lengths(freq, lmax: int = L_MAX):
    """Code lengths (0 for absent symbols) of an optimal prefix code with lengths <= lmax.

    Package-merge: the cost of a length vector is sum(freq * length); an optimal vector under
    the cap is the number of times each symbol appears in the 2n - 2 cheapest items of the list
    obtained by lmax - 1 rounds of "pair up adjacent items of the sorted list, merge the pairs
    with the leaves, sort".  One present symbol gets length 1.
    """
    freq = [int(f) for f in freq]
    syms = [s for s, f in enumerate(freq) if f > 0]
    lengths = [0] * len(freq)
    if not syms:
        return lengths
    if len(syms) == 1:
        lengths[syms[0]] = 1
        return lengths
    if len(syms) > (1 << lmax):
        raise ValueError("too many symbols for the length cap")
    n = len(syms)
    # an item is (weight, tuple of per-symbol counts); leaves sorted by (weight, symbol)
    leaves = sorted(((freq[s], i) for i, s in enumerate(syms)))
    leaf_items = []
    for f, i in leaves:
        cnt = [0] * n
        cnt[i] = 1
        leaf_items.append((f, tuple(cnt)))
    current = list(leaf_items)
    for _ in range(lmax - 1):
        packages = []
        for a in range(0, len(current) - 1, 2):
            wa, ca = current[a]
            wb, cb = current[a + 1]
            packages.append((wa + wb, tuple(x + y for x, y in zip(ca, cb))))
        # stable merge by weight: leaves first on ties
        current = sorted(leaf_items + packages, key=lambda it: it[0])
    chosen = current[:2 * n - 2]
    counts = [0] * n
    for _, c in chosen:
        for i in range(n):
            counts[i] += c[i]
    for i, s in enumerate(syms):
        lengths[s] = counts[i]
    return lengths


def canonical_codes(lengths):
    """Canonical code value (first bit = most significant) of every symbol with length > 0."""
    order = sorted((l, s) for s, l in enumerate(lengths) if l > 0)
    codes = {}
    code, prev = 0, None
    for l, s in order:
        if prev is not None:
            code = (code + 1) << (l - prev)
        else:
            code = 0
        codes[s] = code
        prev = l
    return codes


def _reverse(v: int, l: int) -> int:
    r = 0
    for _ in range(l):
        r = (r << 1) | (v & 1)
        v >>= 1
    return r


def lut(lengths):
    """4,096 entries: the next 12 stream bits (LSB = first bit) -> exponent | length << 8."""
    table = np.full(1 << LUT_BITS, L_MAX << 8, dtype=np.uint16)
    for s, c in canonical_codes(lengths).items():
        l = lengths[s]
        r = _reverse(c, l)
        for hi in range(1 << (LUT_BITS - l)):
            table[r | (hi << l)] = s | (l << 8)
    return table


class EncodedEC:
    """One tensor in the entropy-coded format (all arrays are numpy)."""

    def __init__(self, n, total_bits, lengths, sm, stream, gaps, bases, table):
        self.n, self.total_bits = int(n), int(total_bits)
        self.lengths = list(lengths)
        self.sm, self.stream, self.gaps, self.bases, self.lut = sm, stream, gaps, bases, table

    @property
    def spans(self) -> int:
        return (self.total_bits + SPAN_BITS - 1) // SPAN_BITS

    @property
    def blocks(self) -> int:
        return (self.spans + BLOCK_SPANS - 1) // BLOCK_SPANS

    @property
    def stored_bytes(self) -> int:
        """sm bytes + stream + gaps + bases + table + 256 code lengths."""
        return (self.n + 4 * self.stream.size + 4 * self.gaps.size + 4 * self.bases.size
                + 2 * self.lut.size + 256)


def encode_with_lengths(w, lengths) -> EncodedEC:
    """The format for the given code lengths (which must give every present exponent a code)."""
    e, sm = split(w)
    n = e.size
    codes = canonical_codes(lengths)
    lens = np.array(lengths, dtype=np.int64)
    if n and (lens[e] == 0).any():
        raise ValueError("an exponent present in w has no code")
    rev = np.zeros(256, dtype=np.uint64)
    for s, c in codes.items():
        rev[s] = _reverse(c, lengths[s])
    per = lens[e] if n else np.zeros(0, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(per)[:-1]]) if n else np.zeros(0, dtype=np.int64)
    total = int(per.sum())
    spans = (total + SPAN_BITS - 1) // SPAN_BITS
    # stream: each code's reversed field OR-ed in at its start bit (fields <= 12 bits may straddle
    # a 32-bit word boundary: split into the two words)
    words = np.zeros(2 * spans, dtype=np.uint64)
    if n:
        field = rev[e]
        wi = (starts // 32).astype(np.int64)
        off = (starts % 32).astype(np.uint64)
        lo = (field << off) & np.uint64(0xFFFFFFFF)
        hi = (field << off) >> np.uint64(32)
        np.bitwise_or.at(words, wi, lo)
        has_hi = hi != 0
        np.bitwise_or.at(words, wi[has_hi] + 1, hi[has_hi])
    stream = words.astype(np.uint32)
    # gaps: first code start at or after 64 j (the stream end if none), minus 64 j
    span_starts = np.arange(spans, dtype=np.int64) * SPAN_BITS
    first = np.searchsorted(starts, span_starts, side="left")
    first_start = np.where(first < n, starts[np.minimum(first, max(n - 1, 0))] if n else 0, total)
    gap = (np.minimum(first_start, total) - span_starts).astype(np.uint32)
    if (gap >= 16).any():
        raise AssertionError("gap does not fit 4 bits")
    gaps = np.zeros((spans + 7) // 8, dtype=np.uint32)
    for j in range(8):
        gaps[: (spans - j + 7) // 8] |= gap[j::8] << np.uint32(4 * j)
    blocks = (spans + BLOCK_SPANS - 1) // BLOCK_SPANS
    block_bits = np.arange(blocks, dtype=np.int64) * SPAN_BITS * BLOCK_SPANS
    bases = np.searchsorted(starts, block_bits, side="left").astype(np.uint32)
    return EncodedEC(n, total, lengths, sm, stream, gaps, bases, lut(lengths))


def encode(w) -> EncodedEC:
    e, _ = split(w)
    freq = np.bincount(e, minlength=256)
    return encode_with_lengths(w, optimal_lengths(freq))


def _bit(stream, pos: int) -> int:
    return (int(stream[pos >> 5]) >> (pos & 31)) & 1


def decode(enc: EncodedEC):
    """Bit-by-bit canonical decode (no table): read bits first to last, growing the code value,
    until it equals the code of some symbol of that length."""
    by_len = {}
    for s, c in canonical_codes(enc.lengths).items():
        by_len[(enc.lengths[s], c)] = s
    e = np.zeros(enc.n, dtype=np.uint8)
    pos = 0
    for i in range(enc.n):
        code, l = 0, 0
        while True:
            code = (code << 1) | _bit(enc.stream, pos)
            pos += 1
            l += 1
            if (l, code) in by_len:
                e[i] = by_len[(l, code)]
                break
            if l > L_MAX:
                raise ValueError("invalid code in the stream")
    if pos != enc.total_bits:
        raise ValueError("stream length mismatch")
    return join(e, enc.sm)


def gemv(enc: EncodedEC, rows: int, cols: int, x):
    """(y, absb) in float64: the weights decoded bit by bit, y = W . x and absb = |W| . |x| (the
    scale of the fused GEMV's tolerance)."""
    w = decode(enc).reshape(rows, cols)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return wf @ xf, np.abs(wf) @ np.abs(xf)


def gap_of(enc: EncodedEC, j: int) -> int:
    return (int(enc.gaps[j // 8]) >> (4 * (j % 8))) & 0xF


def decode_span(enc: EncodedEC, j: int):
    """Exponents of the codes that start in span j, decoded from gap[j] with the table."""
    pos = j * SPAN_BITS + gap_of(enc, j)
    end = min((j + 1) * SPAN_BITS, enc.total_bits)
    out = []
    while pos < end:
        window = 0
        for k in range(LUT_BITS):
            p = pos + k
            if p < 32 * enc.stream.size:
                window |= _bit(enc.stream, p) << k
        entry = int(enc.lut[window])
        out.append(entry & 0xFF)
        pos += entry >> 8
    return out


def huffman_cost(freq) -> int:
    """Cost sum(freq * length) of an unconstrained Huffman code (heap of subtree weights)."""
    f = [int(x) for x in freq if x > 0]
    if len(f) <= 1:
        return sum(f)
    heap = list(f)
    heapq.heapify(heap)
    cost = 0
    while len(heap) > 1:
        a = heapq.heappop(heap)
        b = heapq.heappop(heap)
        cost += a + b
        heapq.heappush(heap, a + b)
    return cost


def brute_force_cost(freq, lmax: int) -> int:
    """Minimum of sum(freq * length) over every length vector in [1, lmax]^n with Kraft sum <= 1
    (small n only)."""
    f = [int(x) for x in freq if x > 0]
    if len(f) <= 1:
        return sum(f)
    best = None
    for ls in itertools.product(range(1, lmax + 1), repeat=len(f)):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            c = sum(a * b for a, b in zip(f, ls))
            best = c if best is None else min(best, c)
    return best
