"""Pins for oracle step C-4 (textbook BPE).

* hand-worked tiny merge tables (tests/golden/bpe_hand.json);
* closed form: with merges (a,a)->A1, (A1,A1)->A2, ..., a run of n copies of
  'a' encodes to the binary decomposition of n, largest block first (the
  repeated-character piece of GraphTok, section 6.6, is this shape);
* brute force on every string of up to 8 bytes over {a,b,c} under hand and
  random merge tables, against two independent formulations written here:
  a heap over (rank, position) with a linked list (the "offline heap BPE" the
  centroid-search paper audits against, section 4), and rank-by-rank rounds
  that merge every leftmost non-overlapping occurrence of the round's pair
  (TokTier, section 4, "GPU BPE": the round equivalence);
* every vocabulary string encodes to its own ID.
"""
import heapq
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from tests import vocab

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bpe_hand.json")


def heap_bpe(merges, b: bytes) -> list:
    ranks = {(int(x), int(y)): r for r, (x, y) in enumerate(merges)}
    sym = list(b)
    n = len(sym)
    nxt = list(range(1, n + 1))
    prv = list(range(-1, n - 1))
    alive = [True] * n
    h = []
    for i in range(n - 1):
        r = ranks.get((sym[i], sym[i + 1]))
        if r is not None:
            h.append((r, i))
    heapq.heapify(h)
    while h:
        r, i = heapq.heappop(h)
        if not alive[i] or nxt[i] >= n or ranks.get((sym[i], sym[nxt[i]])) != r:
            continue
        j = nxt[i]
        sym[i] = 256 + r
        alive[j] = False
        nxt[i] = nxt[j]
        if nxt[j] < n:
            prv[nxt[j]] = i
        p = prv[i]
        if p >= 0:
            rp = ranks.get((sym[p], sym[i]))
            if rp is not None:
                heapq.heappush(h, (rp, p))
        k = nxt[i]
        if k < n:
            rk = ranks.get((sym[i], sym[k]))
            if rk is not None:
                heapq.heappush(h, (rk, i))
    out = []
    i = 0 if n else n
    while i < n:
        out.append(sym[i])
        i = nxt[i]
    return out


def rounds_bpe(merges, b: bytes) -> list:
    ranks = {(int(x), int(y)): r for r, (x, y) in enumerate(merges)}
    sym = list(b)
    while True:
        rs = [ranks[(sym[j], sym[j + 1])] for j in range(len(sym) - 1) if (sym[j], sym[j + 1]) in ranks]
        if not rs:
            return sym
        r = min(rs)
        a, c = int(merges[r][0]), int(merges[r][1])
        out, j = [], 0
        while j < len(sym):
            if j + 1 < len(sym) and sym[j] == a and sym[j + 1] == c:
                out.append(256 + r)
                j += 2
            else:
                out.append(sym[j])
                j += 1
        sym = out


def random_table(rng, k: int, alphabet=(97, 98, 99)) -> list:
    pool = list(alphabet)
    seen = set()
    m = []
    while len(m) < k:
        a, b = int(pool[rng.integers(len(pool))]), int(pool[rng.integers(len(pool))])
        if (a, b) in seen:
            continue
        seen.add((a, b))
        m.append((a, b))
        pool.append(255 + len(m))
    return m


def test_hand_examples():
    d = json.load(open(GOLDEN))
    for c in d["cases"]:
        o = oracle.Oracle(d["tables"][c["table"]], "gpt2")
        assert o.bpe(c["text"].encode()) == c["ids"], (c["table"], c["text"], c["why"])


def test_closed_form_repeated_byte():
    k = 6
    m = [(97, 97)] + [(256 + j, 256 + j) for j in range(k - 1)]  # A1..Ak
    o = oracle.Oracle(m, "gpt2")
    for n in list(range(1, 300)) + [1000, 4097, 10_000]:
        want = [256 + k - 1] * (n >> k)
        for j in range(k - 1, -1, -1):
            if (n >> j) & 1:
                want.append(97 if j == 0 else 256 + j - 1)
        assert o.bpe(b"a" * n) == want, n


@pytest.mark.parametrize("table_seed", [None, 1, 2, 3, 4, 5])
def test_brute_force_small_strings(table_seed):
    if table_seed is None:
        m = [(97, 98), (256, 99), (98, 99), (99, 99), (97, 97), (260, 98), (257, 257)]
    else:
        m = random_table(np.random.default_rng(table_seed), 12)
    o = oracle.Oracle(m, "gpt2")
    for n in range(0, 9):
        for tup in itertools.product(b"abc", repeat=n):
            s = bytes(tup)
            got = o.bpe(s)
            assert got == heap_bpe(m, s) == rounds_bpe(m, s), (m, s)


def test_random_longer_against_heap():
    rng = np.random.default_rng(99)
    m = random_table(rng, 60, alphabet=(97, 98, 99, 100))
    o = oracle.Oracle(m, "gpt2")
    for _ in range(3000):
        s = bytes(int(x) for x in rng.integers(97, 101, int(rng.integers(1, 64))))
        assert o.bpe(s) == heap_bpe(m, s) == rounds_bpe(m, s)


@pytest.mark.parametrize("name", ["tiny_1k", "gpt2_50k", "llama3_128k"])
def test_every_vocab_string_encodes_to_its_id(name):
    m = vocab.merges(name)
    tok = vocab.token_bytes(m)
    o = oracle.Oracle(m, "gpt2")
    bad = [v for v in range(256, len(tok)) if o.bpe(tok[v]) != [v]]
    assert not bad, f"{len(bad)} vocabulary strings do not encode to their own ID, e.g. {bad[:5]}"


def test_merge_validation():
    with pytest.raises(oracle.OracleError):
        oracle.Oracle([(97, 256)], "gpt2")  # operand not yet defined
    with pytest.raises(oracle.OracleError):
        oracle.Oracle([(97, 98), (97, 98)], "gpt2")  # duplicate pair
    with pytest.raises(oracle.OracleError):
        oracle.Oracle([], 7)
