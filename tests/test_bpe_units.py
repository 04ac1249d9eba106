"""Units of BPE: a piece splits where no token spans the byte pair.

A merge joins two tokens, so every token that spans a byte boundary holds
that boundary's two bytes.  Where no vocabulary token holds the pair (a, b),
textbook BPE (GraphTok, section 4: lowest rank first, leftmost on ties)
keeps a token boundary there at every step.  The pipeline then merges the
bytes on either side as separate units.  These tests check the claim on the
CPU oracle alone: BPE of a piece equals the concatenated BPE of its units.
They use the pieces of the workloads, CJK-dense text (where units are what
keep long ideograph runs short) and random byte strings over a small
alphabet.  A control shows that cutting at a pair some token does span
changes the result, so the check can fail.
"""
import random

import numpy as np
import pytest

import oracle
from synth import textgen
from tests import libs, vocab


def joinable_pairs(m):
    """Every adjacent byte pair inside the bytes of some token (the definition)."""
    occ = np.zeros((256, 256), dtype=bool)
    for t in vocab.token_bytes(m):
        a = np.frombuffer(t, dtype=np.uint8)
        if len(a) > 1:
            occ[a[:-1], a[1:]] = True
    return occ


def units(piece: bytes, occ) -> list[bytes]:
    cuts = [0] + [i for i in range(1, len(piece)) if not occ[piece[i - 1], piece[i]]] + [len(piece)]
    return [piece[a:b] for a, b in zip(cuts, cuts[1:])]


def unit_bpe(o, piece, occ):
    out = []
    for u in units(piece, occ):
        out += list(o.bpe(u))
    return out


@pytest.mark.parametrize("name", ["gpt2", "llama3", "o200k"])
def test_units_of_workload_pieces(name):
    libs.ensure_built()
    merges_name, pattern = libs.CONFIGS[name]
    m = vocab.merges(merges_name)
    o = oracle.Oracle(m, pattern)
    occ = joinable_pairs(m)
    checked = 0
    for text in (textgen.cjk_text(71, 30_000), textgen.mix_text(72, 60_000)):
        for p in o.piece_strings(text.encode()):
            if len(p) > 1500 or len(units(p, occ)) == 1:
                continue
            assert list(o.bpe(p)) == unit_bpe(o, p, occ), p[:40]
            checked += 1
    assert checked > 30


def test_units_of_random_bytes():
    """Random strings over bytes whose pairs are partly joinable: many cuts,
    and tokens of every length on both sides of them."""
    libs.ensure_built()
    m = vocab.merges("gpt2_50k")
    o = oracle.Oracle(m, "gpt2")
    occ = joinable_pairs(m)
    rng = random.Random(5)
    alpha = b"etaoin sh\xe4\xb8\xad\xe6\x96\x87\x80\xbf"
    cut_cases = 0
    for _ in range(3000):
        p = bytes(rng.choice(alpha) for _ in range(rng.randint(2, 40)))
        if len(units(p, occ)) > 1:
            cut_cases += 1
        assert list(o.bpe(p)) == unit_bpe(o, p, occ), p
    assert cut_cases > 500


def test_cutting_a_joinable_pair_can_change_the_result():
    libs.ensure_built()
    m = vocab.merges("gpt2_50k")
    o = oracle.Oracle(m, "gpt2")
    occ = joinable_pairs(m)
    changed = 0
    for p in o.piece_strings(textgen.mix_text(73, 5_000).encode()):
        for i in range(1, len(p)):
            if occ[p[i - 1], p[i]] and list(o.bpe(p)) != list(o.bpe(p[:i])) + list(o.bpe(p[i:])):
                changed += 1
                break
    assert changed > 50
