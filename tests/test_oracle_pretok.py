"""Pins for oracle step C-3 (the direct leftmost-first pre-tokenizer).

The oracle's cursor matcher is compared with a third, independent matcher: the
``regex`` module running the published alternation for each family (the same
module whose Unicode tables froze the class data).  Exhaustive over a small
alphabet that holds every rule-relevant character kind, then random longer
strings over a wider alphabet, then the full seeded workload texts.  The
worked examples of the pages are in tests/golden/pretok_examples.json.
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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pretok_examples.json")

# letters incl. contraction letters and the long s (folds to 's'), apostrophe,
# U+0020, TAB, LF, CR, NBSP, ASCII digit, superscript two (N), period, CJK
# letter, combining acute (O)
ALPHA_SMALL = ["a", "s", "S", "ſ", "l", "r", "e", "'", " ", "\t", "\n", "\r",
               " ", "1", "²", ".", "中", "́"]
ALPHA_WIDE = ALPHA_SMALL + ["t", "v", "m", "d", "L", "T", "D", "0", "9", "_", '"', "(", "{",
                            "\u0085", " ", "　", "\U0001F600", "é", "١"]


def regex_pieces(pattern: str, s: str) -> list:
    return [p.encode() for p in regex.findall(PATTERNS[pattern], s)]


@pytest.fixture(scope="module", params=["gpt2", "llama3"])
def orc(request):
    return request.param, oracle.Oracle([], request.param)


def test_golden_examples():
    d = json.load(open(GOLDEN))
    for c in d["cases"]:
        o = oracle.Oracle([], c["pattern"])
        got = o.piece_strings(c["text"])
        if "pieces" in c:
            assert got == [p.encode() for p in c["pieces"]], (c["text"], got, c["cite"])
        for p in c.get("contains", []):
            assert p.encode() in got, (c["text"], got, c["cite"])


def test_exhaustive_small_alphabet(orc):
    pat, o = orc
    n_bad = 0
    for n in range(1, 5):
        for tup in itertools.product(ALPHA_SMALL, repeat=n):
            s = "".join(tup)
            if o.piece_strings(s) != regex_pieces(pat, s):
                n_bad += 1
                assert n_bad == 0, (pat, repr(s), o.piece_strings(s), regex_pieces(pat, s))


def test_random_strings(orc):
    pat, o = orc
    rng = np.random.default_rng(11 if pat == "gpt2" else 12)
    for _ in range(20000):
        n = int(rng.integers(1, 40))
        s = "".join(ALPHA_WIDE[i] for i in rng.integers(0, len(ALPHA_WIDE), n))
        assert o.piece_strings(s) == regex_pieces(pat, s), (pat, repr(s))


def test_long_runs(orc):
    pat, o = orc
    for s in ["7" * 1000, " " * 999 + "x", "\n" * 50 + "  " + "y", "'" * 300 + "s", "a" * 5000,
              "x" + " \t" * 200 + "\r\n" * 10 + "  z", "中" * 777, "1" * 3 + "a" + "2" * 7]:
        assert o.piece_strings(s) == regex_pieces(pat, s), (pat, s[:40])


@pytest.mark.parametrize("pat,gen,seed,n", [("gpt2", "tiny", 1, 10_000),
                                            ("gpt2", "mix", 2, 1_000_000),
                                            ("llama3", "mix", 3, 1_000_000)])
def test_workload_text(pat, gen, seed, n):
    text = textgen.tiny_text(seed, n) if gen == "tiny" else textgen.mix_text(seed, n)
    o = oracle.Oracle([], pat)
    assert o.piece_strings(text) == regex_pieces(pat, text)
