"""The piece-start rules of the pre-tokenization kernel (pretok_rules.h),
built for the CPU, against the oracle's direct leftmost-first matcher; and the
closed-form round selection of the long-piece merge kernel against a
sequential definition.

The CPU build runs the very rule functions and scan elements the kernel uses,
sequentially over whole texts, so a rule mistake shows up here without a GPU;
the kernel's scans and tile carries are covered by the GPU parity tests."""
import ctypes
import itertools
import random

import numpy as np
import pytest

import oracle
from exact_byte_level_utf8_amd import build as tkbuild
from synth import textgen
from tests import libs

ALPHA = ["a", "b", "s", "t", "r", "e", "l", "d", "S", "ſ", "'", " ", "\n", "\r", "\t", "1", "2",
         "!", ".", " ", "é", "中", "́", "\U0001F600", "\u0085"]


@pytest.fixture(scope="module")
def rules():
    libs.ensure_built()
    L = ctypes.CDLL(tkbuild.RULES_LIB)
    L.rules_cpu_pieces.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.POINTER(ctypes.c_size_t)]
    L.rules_cpu_select.restype = ctypes.c_uint64
    L.rules_cpu_select.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
    L.rules_cpu_class.argtypes = [ctypes.c_uint32]
    L.rules_cpu_class_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    L.rules_cpu_class_range.restype = None
    L.rules_cpu_fold_extra.argtypes = [ctypes.c_uint32]
    L.rules_cpu_letter_code.argtypes = [ctypes.c_uint32]

    def pieces(b: bytes, pat: int, doc_off=None):
        out = np.zeros(max(len(b), 1), dtype=np.uint64)
        n = ctypes.c_size_t()
        off = None if doc_off is None else np.ascontiguousarray(doc_off, dtype=np.uint64)
        rc = L.rules_cpu_pieces(b, len(b), None if off is None else off.ctypes.data,
                                0 if off is None else off.size - 1, pat, out.ctypes.data, out.size,
                                ctypes.byref(n))
        assert rc == 0
        return out[: n.value].tolist()

    L.pieces = pieces
    return L


@pytest.fixture(scope="module")
def orcs():
    m = np.zeros((0, 2), dtype=np.uint32)
    return [oracle.Oracle(m, "gpt2"), oracle.Oracle(m, "llama3")]


def test_device_class_table_matches_oracle_table(rules):
    """Every Unicode scalar value (U+0000..U+10FFFF without the surrogates):
    the kernels' class table equals the oracle's, which is pinned against the
    regex module code point by code point."""
    n = 0x110000
    dev = np.zeros(n, dtype=np.uint8)
    rules.rules_cpu_class_range(0, n, dev.ctypes.data)
    want = oracle.class_range(0, n)
    scalar = np.ones(n, dtype=bool)
    scalar[0xD800:0xE000] = False
    bad = np.nonzero((dev != want) & scalar)[0]
    assert bad.size == 0, [hex(int(c)) for c in bad[:10]]


def test_device_fold_table(rules):
    """The kernels' non-ASCII contraction letters are exactly the code points
    that the regex module's case-insensitive matching takes for one of the
    contraction letters s t r e v m l d, each mapped to that letter; checked
    over every scalar value outside ASCII."""
    import regex
    any_letter = regex.compile("(?i)[strevmld]")
    singles = {a: regex.compile("(?i)" + a) for a in "strevmld"}
    for cp in range(0x80, 0x110000):
        if 0xD800 <= cp <= 0xDFFF:
            continue
        ch = chr(cp)
        code = rules.rules_cpu_fold_extra(cp)
        if not any_letter.fullmatch(ch):
            assert code == 0, hex(cp)
            continue
        letter = next(a for a, r in singles.items() if r.fullmatch(ch))
        assert code != 0 and code == rules.rules_cpu_letter_code(ord(letter)), hex(cp)


@pytest.mark.parametrize("pat", [0, 1])
def test_exhaustive_short_strings(rules, orcs, pat):
    bad = []
    for n in range(1, 5):
        for tup in itertools.product(ALPHA, repeat=n):
            b = "".join(tup).encode()
            if rules.pieces(b, pat) != orcs[pat].pieces(b):
                bad.append(b)
    assert not bad, bad[:10]


@pytest.mark.parametrize("pat", [0, 1])
def test_random_strings(rules, orcs, pat):
    rng = random.Random(11 + pat)
    for _ in range(30000):
        b = "".join(rng.choice(ALPHA) for _ in range(rng.randint(1, 48))).encode()
        assert rules.pieces(b, pat) == orcs[pat].pieces(b), b


@pytest.mark.parametrize("pat", [0, 1])
def test_long_runs_and_workload(rules, orcs, pat):
    texts = ["7" * 10001 + "x", "x" + " " * 5000 + "y", "a\n" + " " * 3000 + "\n  b", "!" + "\r\n" * 2000 + "  z",
             "'s" * 1000, textgen.mix_text(77, 150_000)]
    for t in texts:
        b = t.encode()
        assert rules.pieces(b, pat) == orcs[pat].pieces(b)


def test_documents_are_hard_boundaries(rules, orcs):
    docs = ["ab", "'s x", "12", "345", "\n", "\n  y", "", "  ", "!\n", "\nq"]
    data = "".join(docs).encode()
    off = np.cumsum([0] + [len(d.encode()) for d in docs])
    for pat in (0, 1):
        want = []
        for d, s in zip(docs, off[:-1]):
            want += [int(s) + p for p in orcs[pat].pieces(d.encode())]
        assert rules.pieces(data, pat, off) == want


def test_round_selection_closed_form(rules):
    def ref(m, carry):
        s, prev = 0, carry
        for j in range(64):
            take = (m >> j) & 1 and not prev
            if take:
                s |= 1 << j
            prev = take
        return s

    rng = random.Random(3)
    for _ in range(50000):
        p = rng.choice([0.1, 0.5, 0.9, 0.99])
        m = sum(1 << j for j in range(64) if rng.random() < p)
        c = rng.randint(0, 1)
        assert rules.rules_cpu_select(m, c) == ref(m, c)


# ---------------------------------------------------------------- case-splitting family
# The segment pre-tokenizer (seg_rules.h), built for the CPU and run the way
# the kernel runs it (1 KiB tiles, segments between synchronizing cuts),
# against the oracle's direct matcher.

CASE_ALPHA = ["A", "S", "ǅ", "a", "s", "t", "e", "ʰ", "中", "́", "ः", "ſ", "'", " ", "\t", "\n", "\r", "1", "."]
CASE_WIDE = CASE_ALPHA + ["T", "L", "D", "r", "v", "m", "l", "d", "E", "R", "V", "M", "é", "É", "ß", "ǈ", "Ω",
                          "ω", "²", "_", '"', "(", " ", "\u0085", "\U0001F600", "⃝", "ー", "ｱ"]


@pytest.fixture(scope="module")
def case_orc():
    return oracle.Oracle(np.zeros((0, 2), dtype=np.uint32), "o200k")


def test_case_table_matches_oracle(rules):
    """The kernels' letter-case table equals the oracle's (which is pinned
    against the regex module) over every scalar value."""
    rules.rules_cpu_case_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    rules.rules_cpu_case_range.restype = None
    dev = np.zeros(0x110000, dtype=np.uint8)
    rules.rules_cpu_case_range(0, 0x110000, dev.ctypes.data)
    want = oracle.subclass_range(0, 0x110000)
    scalar = np.ones(0x110000, dtype=bool)
    scalar[0xD800:0xE000] = False
    bad = np.nonzero((dev != want) & scalar)[0]
    assert bad.size == 0, [hex(int(c)) for c in bad[:10]]


def test_ascii_case_without_the_table(rules):
    """The kernels classify ASCII by arithmetic: equal to the table (and so
    to the oracle) on all 128 code points."""
    rules.rules_cpu_case_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    rules.rules_cpu_case_range.restype = None
    tab = np.zeros(128, dtype=np.uint8)
    rules.rules_cpu_case_range(0, 128, tab.ctypes.data)
    got = [rules.rules_cpu_ascii_case(b) for b in range(128)]
    assert got == tab.tolist()
    assert got == [int(c) for c in oracle.subclass_range(0, 128)]


def test_case_exhaustive_short_strings(rules, case_orc):
    for n in range(1, 5):
        for tup in itertools.product(CASE_ALPHA, repeat=n):
            b = "".join(tup).encode()
            assert rules.pieces(b, 2) == case_orc.pieces(b), b


def test_case_random_strings(rules, case_orc):
    rng = random.Random(21)
    for _ in range(30000):
        b = "".join(rng.choice(CASE_WIDE) * rng.choice([1, 1, 1, 2, 5]) for _ in range(rng.randint(1, 40))).encode()
        assert rules.pieces(b, 2) == case_orc.pieces(b), b


LONG_RUNS = ["A" * 3000 + "b" * 2000 + " x", "ab" * 2000 + "C", "中" * 777 + "A", "7" * 5000 + "x",
             " " * 3000 + "y", "x" + "\n" * 2050 + "  y", "Aa" * 1500, "a" + "́" * 1300 + "B", "DON'T" * 400,
             "'" * 3000 + "s", "!" + "́" * 2000 + "a", "x'd" * 900, "中" + "A" * 4000 + " ", "AB" * 700 + "cd" * 700,
             "\u00a0" * 2000 + "x", " " + "!" * 3000 + "\r\n" * 700 + "z", "中A" * 1500 + "b", "7" * 4001,
             "x" + " " * 1500 + "\n" + " " * 1500 + "y", "a" * 1261 + "B", "A" * 1258 + "'LL x"]


@pytest.mark.parametrize("pat", [2, 3])
def test_case_long_runs_across_tiles(rules, case_orc, pat):
    """Pieces and runs longer than a tile's window, with the tile's cursor
    handed over (2) and recomputed by walking back (3)."""
    for t in LONG_RUNS + [textgen.cjk_text(8, 5000)]:
        for pre in ["", "q", " ", "中" * 5, "x" * 1019, "x" * 1020, "x" * 1021, "x" * 1023]:
            b = (pre + t).encode()
            assert rules.pieces(b, pat) == case_orc.pieces(b), (pre[:3], len(pre), t[:30])


@pytest.mark.parametrize("seed,n", [(2, 150_000), (3, 60_000)])
def test_case_workload_text(rules, case_orc, seed, n):
    b = textgen.mix_text(seed, n).encode()
    assert rules.pieces(b, 2) == case_orc.pieces(b)
    assert rules.pieces(b, 3) == case_orc.pieces(b)


def test_case_documents_are_hard_boundaries(rules, case_orc):
    rng = random.Random(4)
    docs = ["".join(rng.choice(CASE_WIDE) for _ in range(rng.randint(0, 30))) for _ in range(300)]
    docs += ["中" * 900, "7" * 2500, " " * 1800, "A" * 700] * 3
    rng.shuffle(docs)
    data = "".join(docs).encode()
    off = np.cumsum([0] + [len(d.encode()) for d in docs])
    want = []
    for d, s in zip(docs, off[:-1]):
        want += [int(s) + p for p in case_orc.pieces(d.encode())]
    assert rules.pieces(data, 2, off) == want
    assert rules.pieces(data, 3, off) == want


def test_case_scan_alone_matches_the_oracle(rules, case_orc):
    """The forward scan by itself (seg_rules.h: one text, no window, no
    fallback) gives the oracle's pieces, and leaves to the matcher only a
    piece that starts with a mark: on workload text, CJK text, long runs and
    random strings over a case-rich alphabet.  The tile emulation above
    would pass even if the scan handed every piece to the matcher; this
    pins the scan itself."""
    f = rules.rules_cpu_scan_pieces
    f.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.POINTER(ctypes.c_uint64)]
    f.restype = ctypes.c_long

    def check(b: bytes) -> bool:
        out = np.zeros(len(b) + 1, dtype=np.uint64)
        hard = ctypes.c_uint64(0)
        k = f(b, len(b), out.ctypes.data, len(out), ctypes.byref(hard))
        assert k >= 0, b[:60]
        want = case_orc.pieces(b)
        h = hard.value
        assert out[:k].tolist() == [p for p in want if p < h], b[:60]
        if h == len(b):
            return True
        assert h in want, b[:60]
        cp = ord(b[h:h + 4].decode("utf-8", errors="ignore")[0])
        assert int(oracle.subclass_range(cp, 1)[0]) == 3, (hex(cp), b[:60])  # a mark
        return False

    for b in [textgen.mix_text(2, 100_000).encode(), textgen.cjk_text(8, 20_000).encode()] + \
             [t.encode() for t in LONG_RUNS if "\u0301" not in t]:
        check(b)
    rng = random.Random(23)
    whole = 0
    for _ in range(20000):
        b = "".join(rng.choice(CASE_WIDE) * rng.choice([1, 1, 1, 2, 5]) for _ in range(rng.randint(1, 40))).encode()
        whole += check(b)
    assert whole > 5000  # most strings have no piece that starts with a mark
