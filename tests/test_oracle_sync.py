"""Synchronizing transitions, derived by brute force from the CPU oracle.

Append repair accepts a splice only at a stable pre-tokenization boundary
(TokTier, section 3 and Appendix A, Definition A.4).  The library's
certificate is a class change between code points x and y at byte b that it
declares synchronizing (tok_sync_boundary).  This test derives the set from
the oracle's direct leftmost-first matcher alone, with no knowledge of the
library's rules.

A pair (x, y) fails if, for some left context C and right context R, with
S = C x y R and b the byte offset of y:
  (P1) b does not start a piece of S, or the pieces of S from b on differ from
       the pieces of y R shifted by b;
  (P2) for some split R = R1 R2, the pieces of C x y R1 before b differ from
       those of S, or b does not start a piece of C x y R1.
(P1) makes the window's pieces from b on equal the full text's; (P2) makes the
stored text's pieces before b equal the full text's.

The library must declare a pair synchronizing only if it never fails
(soundness).  It must also declare every pair that never fails, so the set is
exact on this alphabet and documents the reading.
"""
import itertools
import random

import pytest

import oracle
from exact_byte_level_utf8_amd import sync_boundary
from tests import libs, vocab

ALPHA = ["s", "e", "l", "r", "t", "a", "S", "é", "1", "2", "²", " ", "\t", "\n", "\r", " ",
         "'", ".", "!", "́", "\U0001F600"]
SMALL = ["s", "e", "1", " ", "\n", "\t", "'", "."]


def _fails(orc, C: str, x: str, y: str, R: str) -> bool:
    S = (C + x + y + R).encode()
    b = len((C + x).encode())
    full = orc.pieces(S)
    if b not in full:
        return True
    suffix = orc.pieces((y + R).encode())
    if [p for p in full if p >= b] != [b + p for p in suffix]:
        return True
    before = [p for p in full if p < b]
    for k in range(len(R) + 1):
        old = orc.pieces((C + x + y + R[:k]).encode())
        if b not in old or [p for p in old if p < b] != before:
            return True
    return False


def _derive(pattern: str, alpha=ALPHA, small=SMALL, klass=lambda c: oracle.char_class(ord(c))):
    orc = oracle.Oracle(vocab.merges("tiny_1k"), pattern)
    cls = {c: klass(c) for c in alpha}
    pairs = [(x, y) for x in alpha for y in alpha if cls[x] != cls[y]]
    ALPHA_, SMALL_ = alpha, small
    rng = random.Random(12345)
    failing = set()
    small_ctx = ["".join(t) for n in range(3) for t in itertools.product(SMALL_, repeat=n)]
    small_right = ["".join(t) for n in range(2) for t in itertools.product(SMALL_, repeat=n)]
    for x, y in pairs:
        done = False
        # exhaustive over short contexts from a smaller alphabet
        for C in small_ctx:
            for R in small_right:
                if _fails(orc, C, x, y, R):
                    failing.add((x, y))
                    done = True
                    break
            if done:
                break
        if done:
            continue
        # random longer contexts from the full alphabet, with runs
        for _ in range(150):
            C = "".join(rng.choice(ALPHA_) * rng.choice([1, 1, 2, 4]) for _ in range(rng.randint(0, 4)))
            R = "".join(rng.choice(ALPHA_) * rng.choice([1, 1, 2, 4]) for _ in range(rng.randint(0, 4)))
            if _fails(orc, C, x, y, R):
                failing.add((x, y))
                break
    return pairs, failing


# the case-splitting family: letters of every case kind, the letters that end
# two-letter contractions in either case, and marks
CASE_ALPHA = ["s", "e", "l", "r", "v", "a", "S", "E", "L", "A", "ǅ", "ʰ", "中", "́", "ः", "é", "1", "²", " ", "\t",
              "\n", "\r", "\u00a0", "'", ".", "!", "\U0001F600"]
CASE_SMALL = ["s", "l", "A", "L", "中", "́", "1", " ", "\n", "'", "."]


@pytest.mark.parametrize("pattern", ["gpt2", "llama3", "o200k"])
def test_sync_set_is_sound_and_exact(pattern):
    libs.ensure_built()
    if pattern == "o200k":
        pairs, failing = _derive(pattern, CASE_ALPHA, CASE_SMALL, lambda c: int(oracle.subclass_range(ord(c), 1)[0]))
    else:
        pairs, failing = _derive(pattern)
    claimed = {(x, y) for x, y in pairs if sync_boundary(pattern, ord(x), ord(y))}
    unsound = sorted(claimed & failing)
    assert not unsound, f"declared synchronizing but the oracle finds a failure: {unsound}"
    missed = sorted(set(pairs) - failing - claimed)
    assert not missed, f"never fails in the oracle but not declared: {missed}"
    # the certificate is useful: most class changes qualify
    assert len(claimed) > len(pairs) // 2


def test_same_class_is_never_a_certificate():
    libs.ensure_built()
    for pattern in ("gpt2", "llama3", "o200k"):
        for x, y in [("a", "b"), (" ", " "), ("1", "2"), (".", "!"), ("\n", " ")]:
            assert not sync_boundary(pattern, ord(x), ord(y))
