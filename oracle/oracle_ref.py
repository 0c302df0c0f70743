"""Literal pure-Python reference for tiny inputs (TEST INFRASTRUCTURE ONLY).

A second, independent reading of the same format, written with Python sets, lists and bit
strings instead of C loops: the codebook is ``sorted(set(w))`` (unsigned 16-bit order), b is the
smallest width with 2**b >= U (0 when U <= 1), and the stream is the concatenation of every index
written as b binary digits least significant first, cut into 32-digit words whose first digit is
bit 0.  Follows the "How it works" section of the codebook lossless compression overview
(dictionary of values + indices, exact substitution back) and the bit-packing of unique-weight
indices described in the Codebook-Quantization digest ("Key points").

Only for small n: everything is Python objects.
"""
from __future__ import annotations

CORRUPT = 0x7FC0


def bits_for(U: int) -> int:
    b = 0
    while 2 ** b < U:
        b += 1
    return b


def encode(w):
    """Return (codebook list, U, b, words list) for a sequence of 16-bit ints."""
    w = [int(v) & 0xFFFF for v in w]
    codebook = sorted(set(w))
    U = len(codebook)
    b = bits_for(U)
    position = {v: i for i, v in enumerate(codebook)}
    digits = "".join(format(position[v], f"0{b}b")[::-1] if b else "" for v in w)
    nwords = (len(digits) + 31) // 32
    digits = digits.ljust(nwords * 32, "0")
    words = [int(digits[32 * k:32 * k + 32][::-1], 2) for k in range(nwords)]
    return codebook, U, b, words


def decode(codebook, b, words, n):
    digits = "".join(format(word, "032b")[::-1] for word in words)
    out = []
    for i in range(n):
        field = digits[i * b:(i + 1) * b]
        idx = int(field[::-1], 2) if b else 0
        out.append(codebook[idx] if idx < len(codebook) else CORRUPT)
    return out


def compressed_bytes(n: int, U: int) -> int:
    """Accounting size: two bytes per codebook entry plus the packed bits rounded up to bytes."""
    b = bits_for(U)
    return 2 * U + (n * b + 7) // 8
