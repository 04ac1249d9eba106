"""Pins for the oracle's case-splitting family (the o200k-style pattern, read
from TokTier, section 4 "Removing the sequential regex scan": the lineage adds
a case-boundary rule to letter runs and a contraction path, and marks take
their own path).

The reading used here: the Llama-3-style alternatives, with the letter
alternative replaced by two that split letter runs at case boundaries
(P? H* T+ S? and P? H+ T* S?, H = upper-case or caseless letters or marks,
T = lower-case or caseless letters or marks, P = one char that is not CR, LF,
a letter or a number) and the contractions moved into an optional suffix S of
a letter piece.  The oracle's cursor matcher (oracle.cpp, o200k_next) is
compared with the third-party ``regex`` module running that alternation
(synth.train_vocab.PATTERNS["o200k"]): the letter-case and mark table
exhaustively, then pieces exhaustively over a small alphabet that holds every
case kind, at random over a wider one, on long runs and on the workload texts.
"""
import itertools
import json
import os

import numpy as np
import pytest
import regex

import oracle
from synth import textgen
from synth.train_vocab import PATTERNS

PAT = "o200k"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pretok_examples.json")

# upper (A, S), title case (U+01C5), lower (a, s, t, e), modifier letter
# (U+02B0), other letter (CJK), non-spacing and spacing marks, long s (folds
# to s), apostrophe, space, TAB, LF, CR, digit, period
ALPHA_SMALL = ["A", "S", "ǅ", "a", "s", "t", "e", "ʰ", "中", "́", "ः", "ſ", "'", " ", "\t", "\n", "\r", "1", "."]
ALPHA_WIDE = ALPHA_SMALL + ["T", "L", "D", "r", "v", "m", "l", "d", "E", "R", "V", "M", "é", "É", "ß", "ǈ",
                            "Ω", "ω", "²", "_", '"', "(", " ", "\u0085", "\U0001F600", "⃝", "ー", "ｱ"]


def regex_pieces(s: str) -> list:
    return [p.encode() for p in regex.findall(PATTERNS[PAT], s)]


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle([], PAT)


def test_subclass_table_matches_regex_exhaustive():
    s = "".join(chr(c) for c in range(0x110000) if not 0xD800 <= c <= 0xDFFF)
    cps = np.array([ord(c) for c in s], dtype=np.int64)
    ref = np.full(0x110000, -1, dtype=np.int8)
    for k, pat in ((4, r"\p{N}+"), (5, r"\s+"), (0, r"[\p{Lu}\p{Lt}]+"), (1, r"\p{Ll}+"),
                   (2, r"[\p{Lm}\p{Lo}]+"), (3, r"\p{M}+")):
        for m in regex.finditer(pat, s):
            ref[cps[m.start():m.end()]] = k
    ref[ref == -1] = 6
    got = oracle.subclass_range(0, 0x110000).astype(np.int8)
    surrogate = (np.arange(0x110000) >= 0xD800) & (np.arange(0x110000) <= 0xDFFF)
    bad = np.nonzero((ref != got) & ~surrogate)[0]
    assert bad.size == 0, [hex(int(c)) for c in bad[:10]]
    # every letter has a case class, and the four-class table agrees on letters
    cls = np.array([oracle.char_class(c) for c in range(0, 0x3400)])
    assert np.array_equal(cls == 0, got[:0x3400] <= 2)


def test_golden_examples(o):
    d = json.load(open(GOLDEN))
    cases = [c for c in d["cases"] if c["pattern"] == PAT]
    assert len(cases) >= 5
    for c in cases:
        got = o.piece_strings(c["text"])
        assert got == [p.encode() for p in c["pieces"]], (c["text"], got, c["cite"])


def test_exhaustive_small_alphabet(o):
    for n in range(1, 5):
        for tup in itertools.product(ALPHA_SMALL, repeat=n):
            s = "".join(tup)
            assert o.piece_strings(s) == regex_pieces(s), repr(s)


def test_random_strings(o):
    rng = np.random.default_rng(13)
    for _ in range(30000):
        n = int(rng.integers(1, 48))
        s = "".join(ALPHA_WIDE[i] for i in rng.integers(0, len(ALPHA_WIDE), n))
        assert o.piece_strings(s) == regex_pieces(s), repr(s)


def test_long_runs(o):
    for s in ["A" * 3000 + "b" * 2000, "ab" * 2000 + "C", "中" * 777 + "A", "7" * 1000, " " * 999 + "x",
              "x" + "\n" * 50 + "  y", "Aa" * 1500, "a" + "́" * 300 + "B", "DON'T" * 200, "'" * 300 + "s"]:
        assert o.piece_strings(s) == regex_pieces(s), s[:40]


@pytest.mark.parametrize("gen,seed,n", [("mix", 2, 1_000_000), ("cjk", 5, 100_000)])
def test_workload_text(o, gen, seed, n):
    text = textgen.mix_text(seed, n) if gen == "mix" else textgen.cjk_text(seed, n)
    assert o.piece_strings(text) == regex_pieces(text)
