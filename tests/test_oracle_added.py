"""Pins of the oracle's added-token literal pass (oracle.encode_added).

- Hand-worked cases (tests/golden/added_tokens.json, each with its derivation).
- Brute force: on random short texts over a small alphabet with random
  literal sets, the literal selection equals the one Python's `re` makes with
  an alternation of the literals sorted longest first (at each position the
  engine tries the alternatives in order, so the first that matches is the
  longest, and finditer moves left to right over non-overlapping matches:
  leftmost-longest, written independently of the oracle's cursor loop); the
  segments between literals are encoded with the oracle's plain encode.
- A text with no literal occurrence encodes exactly as without literals, and
  malformed UTF-8 is still rejected.
"""
import json
import os
import random
import re

import numpy as np
import pytest

import oracle
from synth import textgen
from tests import vocab

HERE = os.path.dirname(os.path.abspath(__file__))


def load_cases():
    return json.load(open(os.path.join(HERE, "golden", "added_tokens.json")))["cases"]


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: repr(c["text"]))
def test_hand_worked(case):
    o = oracle.Oracle(np.asarray(case["merges"], dtype=np.uint32).reshape(-1, 2), case["pattern"])
    lits = [(s.encode(), i) for s, i in case["literals"]]
    assert o.encode_added(case["text"].encode(), lits).tolist() == case["ids"], case["why"]


def re_reference(o, b: bytes, lits):
    alts = sorted(lits, key=lambda x: -len(x[0]))
    rx = re.compile(b"|".join(re.escape(x) for x, _ in alts))
    ids_of = {}
    for x, i in lits:
        ids_of.setdefault(x, i)  # a repeated string keeps its first ID, as in the cursor scan
    out, seg = [], 0
    for m in rx.finditer(b):
        out += o.encode(b[seg:m.start()]).tolist()
        out.append(ids_of[m.group(0)])
        seg = m.end()
    out += o.encode(b[seg:]).tolist()
    return out


@pytest.mark.parametrize("pattern", ["gpt2", "llama3"])
def test_brute_force_against_re(pattern):
    m = vocab.merges("tiny_1k")
    o = oracle.Oracle(m, pattern)
    rng = random.Random(11)
    alphabet = ["a", "b", "<", "|", ">", "e", " ", "1", "\n", "é"]
    for trial in range(400):
        n_lit = rng.randint(1, 5)
        lits, seen = [], set()
        for k in range(n_lit):
            s = "".join(rng.choice(alphabet) for _ in range(rng.randint(1, 4))).encode()
            if s in seen:
                continue
            seen.add(s)
            lits.append((s, 5000 + k))
        for _ in range(5):
            b = "".join(rng.choice(alphabet) for _ in range(rng.randint(0, 24))).encode()
            assert o.encode_added(b, lits).tolist() == re_reference(o, b, lits), (b, lits)


def test_no_occurrence_is_plain_encode():
    m = vocab.merges("gpt2_50k")
    o = oracle.Oracle(m, "gpt2")
    b = textgen.mix_text(12, 30_000).encode()
    lits = [(b"<|endoftext|>", 50_256 + 1000), (b"<|im_start|>", 50_256 + 1001)]
    assert np.array_equal(o.encode_added(b, lits), o.encode(b))
    with pytest.raises(UnicodeDecodeError):
        o.encode_added(b"ok \xff <|endoftext|>", lits)
