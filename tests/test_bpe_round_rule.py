"""The merge-round rule of the piece pass, emulated on the CPU and checked
against the oracle's textbook BPE (lowest rank first, leftmost on ties).

A round of the piece pass merges at once every pair that is either of the
lowest rank left in its piece, or sheltered.  A pair (x, y) of rank r is
sheltered when both of its sides are:
  left:  walking left from x over at most two more pairs, every pair passed
         ranks above r, and the walk ends at a token t that is never the right
         operand of a merge ranked below r (t = x counts), or at the piece
         start;
  right: the same to the right of y, with tokens that are never the left
         operand of a merge ranked below r.
No merge ranked below r can then reach x or y, so textbook BPE merges (x, y)
before anything changes them, and merging it early leaves the result alone.
Equal-rank runs keep the leftmost non-overlapping pairs.  The claim is
pinned here against oracle.Oracle.bpe on random merge tables over small
alphabets (many interacting merges, long chains) and on the pieces of the
synthetic workloads under the trained vocabularies.

The long-piece kernel uses the same rule with walks of up to 64 pairs (the
argument does not depend on the walk's length); that rule is pinned the same
way, on longer random pieces and on the CJK-dense workload's pieces, where it
cuts the rounds from hundreds to under twenty.  Rules with a planted mistake
(a walk that does not stop at a pair ranked at or below r, or a walk that
takes any token as a barrier) must fail these checks.
"""
import random

import numpy as np

import oracle
from synth import textgen
from tests import vocab

INF = 1 << 40
WALK = 2  # pairs walked past the pair itself on each side


class RuleBPE:
    """BPE of single pieces by rounds of the piece pass's rule."""

    def __init__(self, merges, walk: int = WALK, mistake: str | None = None):
        self.walk = walk
        self.mistake = mistake
        self.rank = {(int(a), int(b)): r for r, (a, b) in enumerate(merges)}
        n_tok = 256 + len(merges)
        self.min_l = [INF] * n_tok  # lowest rank of a merge with the token as right operand
        self.min_r = [INF] * n_tok  # ... as left operand
        for r, (a, b) in enumerate(merges):
            self.min_r[int(a)] = min(self.min_r[int(a)], r)
            self.min_l[int(b)] = min(self.min_l[int(b)], r)

    def __call__(self, piece: bytes, shelter: bool = True) -> tuple[list[int], int]:
        """(ids, rounds); shelter=False merges only the lowest-rank pairs."""
        rank, min_l, min_r = self.rank, self.min_l, self.min_r
        sym = list(piece)
        rounds = 0
        while True:
            pr = [rank.get((sym[i], sym[i + 1]), INF) for i in range(len(sym) - 1)]
            if not pr or min(pr) >= INF:
                return sym, rounds
            rounds += 1
            low = min(pr)
            safe = []
            for i, r in enumerate(pr):
                if r >= INF or (r != low and not shelter):
                    safe.append(False)
                    continue
                if r == low:
                    safe.append(True)
                    continue
                stops = self.mistake != "no_stop"
                barrier = (lambda t, m: True) if self.mistake == "any_barrier" else (lambda t, m: m[t] > r)
                ok_l = barrier(sym[i], min_l)
                for d in range(1, self.walk + 1):
                    if ok_l:
                        break
                    j = i - d
                    if j < 0:
                        ok_l = True
                        break
                    if stops and pr[j] <= r:
                        break
                    ok_l = barrier(sym[j], min_l)
                ok_r = barrier(sym[i + 1], min_r)
                for d in range(1, self.walk + 1):
                    if ok_r:
                        break
                    j = i + d
                    if j >= len(pr):
                        ok_r = True
                        break
                    if stops and pr[j] <= r:
                        break
                    ok_r = barrier(sym[j + 1], min_r)
                safe.append(ok_l and ok_r)
            # adjacent sheltered pairs always have equal rank; keep the
            # leftmost non-overlapping ones
            out, i = [], 0
            while i < len(sym):
                if i < len(pr) and safe[i]:
                    out.append(256 + pr[i])
                    i += 2
                else:
                    out.append(sym[i])
                    i += 1
            sym = out


def random_merges(rng: random.Random, alphabet: bytes, n: int) -> np.ndarray:
    """A merge table over the alphabet: each merge joins two existing tokens."""
    toks = list(alphabet)
    seen = set()
    out = []
    while len(out) < n:
        a, b = rng.choice(toks), rng.choice(toks)
        if (a, b) in seen:
            continue
        seen.add((a, b))
        out.append((a, b))
        toks.append(256 + len(out) - 1)
        # later merges favour recent tokens, so chains grow long
        if rng.random() < 0.5:
            toks.append(256 + len(out) - 1)
    return np.asarray(out, dtype=np.uint32)


def token_bytes(merges, alphabet_tok: int) -> list[bytes]:
    out = [bytes([i]) for i in range(256)]
    for a, b in merges:
        out.append(out[int(a)] + out[int(b)])
    return out


def test_rule_matches_textbook_bpe_on_random_tables():
    rng = random.Random(2026)
    checked = 0
    for t in range(120):
        alphabet = bytes(rng.sample(b"abcdefgh", rng.randint(2, 7)))
        merges = random_merges(rng, alphabet, rng.randint(5, 200))
        toks = token_bytes(merges, 256)[256:]
        orc = oracle.Oracle(merges, "gpt2")
        rule = RuleBPE(merges)
        for i in range(60):
            if i % 2:
                piece = bytes(rng.choice(alphabet) for _ in range(rng.randint(2, 48)))
            else:  # strings of whole tokens, so that deep merges take place
                piece = b"".join(rng.choice(toks) for _ in range(rng.randint(2, 6)))[:64]
            got, _ = rule(piece)
            assert got == orc.bpe(piece), (t, piece, merges.tolist())
            checked += 1
    assert checked == 7200


def test_chains_that_reach_a_pair_from_either_side():
    """Merges ranked below r that reach x or y only after an earlier merge
    next to them: the walk must stop at the lower-ranked pair it meets."""
    v, w, x, y = b"vwxy"
    cases = [
        # (v w) then (W x) takes x before (x y)
        ([(v, w), (256, x), (x, y)], b"vwxy", [257, y]),
        # (w v) then (y W) takes y before (x y)
        ([(w, v), (y, 256), (x, y)], b"xywv", [x, 257]),
        # the same two steps further out, and a barrier that does hold
        ([(v, w), (256, w), (257, x), (x, y)], b"vwwxy", [258, y]),
        ([(x, y), (v, w)], b"vwxy", [257, 256]),
    ]
    for merges, piece, want in cases:
        m = np.asarray(merges, dtype=np.uint32)
        assert oracle.Oracle(m, "gpt2").bpe(piece) == want
        assert RuleBPE(m)(piece)[0] == want


def test_rule_matches_textbook_bpe_on_workload_pieces():
    for merges_name, pattern, seed in (("gpt2_50k", "gpt2", 2), ("llama3_128k", "llama3", 3)):
        m = vocab.merges(merges_name)
        orc = oracle.Oracle(m, pattern)
        rule = RuleBPE(m)
        text = textgen.mix_text(seed, 60_000).encode()
        pieces = sorted(set(orc.piece_strings(text)), key=lambda p: (-len(p), p))
        fewer = 0
        for p in pieces[:800]:
            got, r_rule = rule(p)
            assert got == orc.bpe(p), p
            _, r_text = rule(p, shelter=False)
            fewer += r_rule < r_text
        assert fewer > 100  # the rule shortens many of the longest pieces' chains


LONG_WALK = 64  # the long-piece kernel's walk bound


def test_long_walk_rule_matches_textbook_bpe_on_random_tables():
    rng = random.Random(2027)
    for t in range(80):
        alphabet = bytes(rng.sample(b"abcdefgh", rng.randint(2, 7)))
        merges = random_merges(rng, alphabet, rng.randint(5, 300))
        toks = token_bytes(merges, 256)[256:]
        orc = oracle.Oracle(merges, "gpt2")
        rule = RuleBPE(merges, walk=LONG_WALK)
        for i in range(30):
            if i % 2:
                piece = bytes(rng.choice(alphabet) for _ in range(rng.randint(65, 400)))
            else:
                piece = b"".join(rng.choice(toks) for _ in range(rng.randint(8, 40)))[:400]
            assert rule(piece)[0] == orc.bpe(piece), (t, piece, merges.tolist())


def test_long_walk_rule_on_cjk_pieces():
    """The CJK-dense workload's long pieces: the 64-pair walk gives textbook
    BPE's tokens in far fewer rounds than the two-pair walk."""
    m = vocab.merges("gpt2_50k")
    orc = oracle.Oracle(m, "gpt2")
    short, long_ = RuleBPE(m), RuleBPE(m, walk=LONG_WALK)
    text = textgen.cjk_text(5, 40_000).encode()
    pieces = sorted((p for p in orc.piece_strings(text) if 64 < len(p) <= 1600), key=len)
    assert len(pieces) >= 20
    most_long = most_short = 0
    for p in pieces[:: max(1, len(pieces) // 20)]:
        want = orc.bpe(p)
        got, r_long = long_(p)
        assert got == want, len(p)
        got2, r_short = short(p)
        assert got2 == want
        most_long, most_short = max(most_long, r_long), max(most_short, r_short)
    assert most_long <= 20 < most_short


def test_planted_rule_mistakes_fail():
    """Each planted mistake in the walk gives a wrong result on some random
    table, so the checks above would catch it."""
    for mistake in ("no_stop", "any_barrier"):
        rng = random.Random(2028)
        wrong = 0
        for t in range(80):
            alphabet = bytes(rng.sample(b"abcdefgh", rng.randint(2, 5)))
            merges = random_merges(rng, alphabet, rng.randint(20, 200))
            toks = token_bytes(merges, 256)[256:]
            orc = oracle.Oracle(merges, "gpt2")
            rule = RuleBPE(merges, walk=LONG_WALK, mistake=mistake)
            for _ in range(20):
                piece = b"".join(rng.choice(toks) for _ in range(rng.randint(4, 20)))[:200]
                wrong += rule(piece)[0] != orc.bpe(piece)
        assert wrong > 0, mistake
