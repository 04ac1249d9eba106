"""Pins for oracle steps C-1 (UTF-8 decode) and C-2 (character classes).

C-2 is pinned exhaustively against the third-party ``regex`` module, scanned
with run-finding searches over a string holding every scalar value; C-1 is
pinned against Python's strict UTF-8 codec on random valid and invalid bytes.
"""
import numpy as np
import pytest
import regex

import oracle

L, N, W, O = 0, 1, 2, 3


def _all_scalars() -> str:
    return "".join(chr(c) for c in range(0x110000) if not 0xD800 <= c <= 0xDFFF)


def _regex_classes() -> np.ndarray:
    s = _all_scalars()
    cps = np.array([ord(c) for c in s], dtype=np.int64)
    cls = np.full(0x110000, O, dtype=np.int8)
    for k, pat in ((L, r"\p{L}+"), (N, r"\p{N}+"), (W, r"\s+")):
        for m in regex.finditer(pat, s):
            cls[cps[m.start():m.end()]] = k
    return cls


def test_class_table_matches_regex_exhaustive():
    ref = _regex_classes()
    got = np.array([oracle.char_class(c) for c in range(0x110000)], dtype=np.int8)
    surrogate = (np.arange(0x110000) >= 0xD800) & (np.arange(0x110000) <= 0xDFFF)
    bad = np.nonzero((ref != got) & ~surrogate)[0]
    assert bad.size == 0, f"{bad.size} code points differ, first {[hex(x) for x in bad[:10]]}"


def test_class_spot_values():
    # whitespace set is White_Space (25 code points), not str.isspace
    assert oracle.char_class(0x20) == W and oracle.char_class(0xA0) == W
    assert oracle.char_class(0x85) == W and oracle.char_class(0x3000) == W
    assert oracle.char_class(0x1C) == O  # isspace() says True, White_Space says no
    assert oracle.char_class(ord("²")) == N and oracle.char_class(ord("½")) == N
    assert oracle.char_class(0x0301) == O  # combining mark is not a letter
    assert oracle.char_class(ord("中")) == L and oracle.char_class(0x1F600) == O
    assert oracle.char_class(ord("'")) == O and oracle.char_class(ord("_")) == O
    wset = [c for c in range(0x110000) if oracle.char_class(c) == W]
    assert len(wset) == 25


def _oracle_accepts(o, b: bytes) -> bool:
    try:
        o.encode(b)
        return True
    except UnicodeDecodeError:
        return False


def _codec_accepts(b: bytes) -> bool:
    try:
        b.decode("utf-8", errors="strict")
        return True
    except UnicodeDecodeError:
        return False


def test_utf8_validation_matches_strict_codec():
    o = oracle.Oracle([], "gpt2")
    rng = np.random.default_rng(7)
    special = [b"\xc0\x80", b"\xc1\xbf", b"\xe0\x80\x80", b"\xe0\x9f\xbf", b"\xed\xa0\x80",
               b"\xed\x9f\xbf", b"\xf0\x8f\xbf\xbf", b"\xf4\x90\x80\x80", b"\xf4\x8f\xbf\xbf",
               b"\xf5\x80\x80\x80", b"\xff", b"\x80", b"\xe2\x82", b"a\xc3", b"\xf0\x9f\x98\x80",
               "\U0010FFFF".encode(), "�".encode(), b"\xef\xbf\xbf"]
    cases = list(special)
    for _ in range(20000):
        n = int(rng.integers(1, 7))
        if rng.random() < 0.5:
            cases.append(bytes(rng.integers(0, 256, n, dtype=np.uint8)))
        else:
            pool = [0x41, 0x80, 0xBF, 0xC2, 0xDF, 0xE0, 0xED, 0xEF, 0xF0, 0xF4, 0x9F, 0xA0, 0x8F, 0x90]
            cases.append(bytes(int(pool[i]) for i in rng.integers(0, len(pool), n)))
    for b in cases:
        assert _oracle_accepts(o, b) == _codec_accepts(b), b
