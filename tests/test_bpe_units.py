"""Units of BPE: a piece splits where no token can span the boundary.

A merge joins two tokens, so every token that spans a byte boundary holds
that boundary's two bytes.  Where no vocabulary token holds the pair (a, b),
textbook BPE (GraphTok, section 4: lowest rank first, leftmost on ties)
keeps a token boundary there at every step.  The pipeline then merges the
bytes on either side as separate units.  A finer cut uses the bytes around
the boundary too: a token spanning the boundary between bytes i - 1 and i
is those two bytes alone, or it holds the three bytes i - 2 .. i or the
three bytes i - 1 .. i + 1; where the vocabulary has no such two-byte token
and no token holds either three-byte string, nothing spans the boundary.
These tests check both rules on the CPU oracle alone: BPE of a piece equals
the concatenated BPE of its units.  They use the pieces of the workloads,
CJK-dense text (where units are what keep long ideograph runs short) and
random byte strings over a small alphabet.  Controls show that cutting where
a token does span changes the result, so the checks can fail.
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


def spanning_strings(m):
    """The vocabulary's two-byte tokens, and every three-byte string inside
    some token (the definitions)."""
    two, three = set(), set()
    for t in vocab.token_bytes(m):
        if len(t) == 2:
            two.add(t)
        for i in range(len(t) - 2):
            three.add(t[i:i + 3])
    return two, three


def context_cut(piece: bytes, i: int, occ, two, three) -> bool:
    """No token can span the boundary before byte i of the piece."""
    if not occ[piece[i - 1], piece[i]]:
        return True
    if piece[i - 1:i + 1] in two:
        return False
    left = i >= 2 and piece[i - 2:i + 1] in three
    right = i + 1 < len(piece) and piece[i - 1:i + 2] in three
    return not left and not right


def context_units(piece: bytes, occ, two, three) -> list[bytes]:
    cuts = [0] + [i for i in range(1, len(piece)) if context_cut(piece, i, occ, two, three)] + [len(piece)]
    return [piece[a:b] for a, b in zip(cuts, cuts[1:])]


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


@pytest.mark.parametrize("name", ["gpt2", "llama3", "o200k"])
def test_context_units_of_workload_pieces(name):
    libs.ensure_built()
    merges_name, pattern = libs.CONFIGS[name]
    m = vocab.merges(merges_name)
    o = oracle.Oracle(m, pattern)
    occ = joinable_pairs(m)
    two, three = spanning_strings(m)
    checked = finer = 0
    for text in (textgen.cjk_text(74, 20_000), textgen.mix_text(75, 40_000)):
        for p in o.piece_strings(text.encode()):
            if len(p) > 1500:
                continue
            us = context_units(p, occ, two, three)
            if len(us) == 1:
                continue
            got = []
            for u in us:
                got += list(o.bpe(u))
            assert list(o.bpe(p)) == got, p[:40]
            checked += 1
            finer += len(us) > len(units(p, occ))
    assert checked > 30 and finer > 10


def test_context_units_of_random_bytes():
    """Random strings over a small alphabet with ideograph bytes: dense cuts
    by both rules, and tokens of every length on both sides of them."""
    libs.ensure_built()
    for name in ("gpt2_50k", "o200k_64k"):
        m = vocab.merges(name)
        o = oracle.Oracle(m, "gpt2")
        occ = joinable_pairs(m)
        two, three = spanning_strings(m)
        rng = random.Random(6)
        alpha = b"etaoin sh\xe4\xb8\xad\xe6\x96\x87\x80\xbf\xe5\x9c\xb0"
        cut_cases = 0
        for _ in range(3000):
            p = bytes(rng.choice(alpha) for _ in range(rng.randint(2, 40)))
            us = context_units(p, occ, two, three)
            if len(us) > len(units(p, occ)):
                cut_cases += 1
            got = []
            for u in us:
                got += list(o.bpe(u))
            assert list(o.bpe(p)) == got, (name, p)
        assert cut_cases > 300, cut_cases


def test_cutting_where_a_token_spans_can_change_the_result():
    """Control for the context rule: a boundary it keeps (some two-byte token
    or three-byte string could span it) does change the result when cut."""
    libs.ensure_built()
    m = vocab.merges("gpt2_50k")
    o = oracle.Oracle(m, "gpt2")
    occ = joinable_pairs(m)
    two, three = spanning_strings(m)
    changed = 0
    for p in o.piece_strings(textgen.cjk_text(76, 3_000).encode() + textgen.mix_text(77, 3_000).encode()):
        for i in range(1, len(p)):
            if not context_cut(p, i, occ, two, three) and list(o.bpe(p)) != list(o.bpe(p[:i])) + list(o.bpe(p[i:])):
                changed += 1
                break
    assert changed > 50
