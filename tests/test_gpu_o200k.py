"""GPU parity of the case-splitting (o200k-style) family against the oracle.

The family (TokTier, section 4, "Removing the sequential regex scan": the
o200k lineage adds a case-boundary rule inside letter runs, a contraction
path, and a narrow fallback for marks) is pre-tokenized on the GPU by
segments between synchronizing cuts, each matched from its cut.  Pieces are
compared before IDs (TokTier, section 5.2: split-level checks catch divisions
that identical IDs can hide), then IDs under a merge list trained for the
family, on seeded random strings over a case-rich alphabet (each string its
own document in one batch), runs longer than the kernel's loaded window,
the 1M-char workload, CJK text, documents, malformed input, append repair
(host and device) and span export.
"""
import random

import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, oracle_par, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALPHA = ["A", "S", "ǅ", "a", "s", "t", "e", "r", "v", "l", "E", "L", "ʰ", "中", "́", "ः", "ſ", "'", " ", "\t", "\n",
         "\r", "1", "²", ".", "!", "é", "É", "\U0001F600", " ", "_"]


@pytest.fixture(scope="module")
def cfg():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    merges_name, pattern = libs.CONFIGS["o200k"]
    m = vocab.merges(merges_name)
    return tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern), vocab.token_bytes(m)


def dev_bytes(b: bytes):
    return torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda() if b else torch.empty(0, dtype=torch.uint8,
                                                                                         device="cuda")


def gpu_pieces(t, b: bytes, doc_off=None):
    d = dev_bytes(b)
    flags = torch.zeros((len(b) + 15) // 16 + 8, dtype=torch.int16, device="cuda")
    doc = None if doc_off is None else torch.tensor(np.asarray(doc_off, dtype=np.int64), device="cuda").view(
        torch.uint64)
    t.pretokenize_dev(d, flags, doc)
    torch.cuda.synchronize()
    return tk.flags_to_starts(flags.cpu().numpy().view(np.uint16), len(b)).tolist()


def same(what, got, want):
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape or not np.array_equal(got, want):
        n = min(len(got), len(want))
        i = next((k for k in range(n) if got[k] != want[k]), n)
        pytest.fail(f"{what}: {len(got)} vs {len(want)}, first difference at {i}: "
                    f"gpu {got[i:i + 6].tolist()} oracle {want[i:i + 6].tolist()}")


def random_docs(seed, count, longest):
    rng = random.Random(seed)
    return ["".join(rng.choice(ALPHA) * rng.choice([1, 1, 1, 2, 5]) for _ in range(rng.randint(0, longest)))
            for _ in range(count)]


def test_random_strings_split_and_ids(cfg):
    t, o, _ = cfg
    docs = random_docs(31, 20000, 24)
    data, off = textgen.pack_docs(docs)
    want = []
    for d, s in zip(docs, off[:-1]):
        want += [int(s) + p for p in o.pieces(d.encode())]
    same("pieces", gpu_pieces(t, data, off), want)
    ids, out_off = t.encode_batch(data, off)
    want_ids, want_off = oracle_par.concat(oracle_par.map_docs(lambda d: o.encode(d.encode()), docs))
    same("ids", ids, want_ids)
    same("offsets", out_off, want_off)


def test_one_long_random_text(cfg):
    """The same alphabet as one request: cuts, tiles and halos meet every
    kind of segment."""
    t, o, _ = cfg
    b = "".join(random_docs(32, 4000, 40)).encode()
    same("pieces", gpu_pieces(t, b), o.pieces(b))
    same("ids", t.encode(b), o.encode(b))


@pytest.mark.parametrize("text", [
    "A" * 3000 + "b" * 2000 + " x", "ab" * 2000 + "C", "中" * 777 + "A", "7" * 5000 + "x", " " * 3000 + "y",
    "x" + "\n" * 2050 + "  y", "Aa" * 1500, "a" + "́" * 1300 + "B", "DON'T" * 400, "'" * 3000 + "s",
    "!" + "́" * 2000 + "a", "x'd" * 900, "AB" * 700 + "cd" * 700,
])
def test_runs_longer_than_the_window(cfg, text):
    t, o, _ = cfg
    b = ("pre " + text + " post").encode()
    same("pieces", gpu_pieces(t, b), o.pieces(b))
    same("ids", t.encode(b), o.encode(b))


@pytest.mark.parametrize("gen,seed,n", [("mix", 91, 1_000_000), ("cjk", 92, 40_000), ("mix", 93, 3_000)])
def test_workload(cfg, gen, seed, n):
    t, o, tokb = cfg
    b = (textgen.mix_text(seed, n) if gen == "mix" else textgen.cjk_text(seed, n)).encode()
    same("pieces", gpu_pieces(t, b), o.pieces(b))
    want = o.encode(b)
    same("ids", t.encode(b), want)
    d = dev_bytes(b)
    ids = torch.empty(len(b), dtype=torch.int32, device="cuda")
    k = t.encode_dev(d, ids)
    torch.cuda.synchronize()
    same("device ids", ids[:k].cpu().numpy(), want)


def test_batch_documents(cfg):
    t, o, _ = cfg
    docs = [textgen.mix_text(100 + i, 20_000 + 977 * i) for i in range(16)] + ["", "A", "aB", "x'S"]
    data, off = textgen.pack_docs(docs)
    ids, out_off = t.encode_batch(data, off)
    want_ids, want_off = oracle_par.concat(oracle_par.map_docs(lambda d: o.encode(d.encode()), docs))
    same("ids", ids, want_ids)
    same("offsets", out_off, want_off)


def test_malformed_utf8_rejected(cfg):
    t, _, _ = cfg
    for bad in [b"\xff", b"ab\xc3", b"\xe0\x80\x80", b"\xed\xa0\x80x", b"a\x80b", b"x" * 3000 + b"\xf5\x80\x80\x80"]:
        with pytest.raises(tk.TokError) as e:
            t.encode(bad)
        assert e.value.code == tk.TOK_E_UTF8, bad


def test_spans(cfg):
    t, o, _ = cfg
    b = textgen.mix_text(94, 200_000).encode()
    d = dev_bytes(b)
    ids = torch.empty(len(b), dtype=torch.int32, device="cuda")
    sp = torch.empty(len(b), dtype=torch.int32, device="cuda")
    k = t.encode_spans_dev(d, ids, sp)
    torch.cuda.synchronize()
    want_ids, want_sp = o.encode_spans(b)
    same("ids", ids[:k].cpu().numpy(), want_ids)
    same("spans", sp[:k].cpu().numpy().view(np.uint32).astype(np.uint64), want_sp)


def test_repair(cfg):
    """Appends to a 300K-char context (seam shapes of the family: a word cut
    mid-run, camelCase across the seam, a contraction across it): the host
    and device repairs equal the oracle's full encode."""
    t, o, _ = cfg
    base = textgen.mix_text(95, 300_000)
    cases = [textgen.repair_case(95, 9_700 + i, old_text=base) for i in range(10)]
    cases += [(base + "camel", "Case and more"), (base + "don", "'t stop"), (base + "HTTP", "Server x"),
              (base + "x'", "LL done")]
    for old, suf in cases:
        ob, text = old.encode(), (old + suf).encode()
        sess = o.encode(ob)
        want = o.encode(text)
        got, info = t.repair(sess, text, len(ob))
        same(f"repair {suf[:10]!r}", got, want)
        buf = torch.from_numpy(np.concatenate([sess, np.zeros(len(want) + 8, np.int32)])).cuda()
        n, dinfo = t.repair_dev(buf, len(sess), text, len(ob))
        assert dinfo == info
        same(f"device repair {suf[:10]!r}", buf[:n].cpu().numpy(), want)


# Stretches without a synchronizing cut, a megabyte and more: each tile takes
# the cursor its predecessor hands over, and pieces past the loaded window are
# matched by the whole workgroup.  Split-level parity (the oracle's textbook
# BPE of a megabyte-long piece is quadratic); the IDs of such pieces are
# covered by the long-piece tests of the merge stage.
@pytest.mark.parametrize("text", [
    "中" * 350_000, "7" * 1_000_001, " " * 700_000 + "x", "x'd" * 300_000, "!" * 900_000 + "\n" * 3000 + "a",
    "A" * 600_000 + "b" * 400_000, "中" + "A" * 800_000 + " y", " " * 400_000 + "z",
])
def test_megabyte_stretches_without_a_cut(cfg, text):
    t, o, _ = cfg
    b = ("pre " + text + " post").encode()
    same("pieces", gpu_pieces(t, b), o.pieces(b))


def test_long_runs_inside_batch_documents(cfg):
    """Cut-free runs that start and end inside documents of a batch, cross
    tiles, and meet document boundaries (hard boundaries for the hand-over)."""
    t, o, _ = cfg
    rng = random.Random(33)
    kinds = ["中", "7", " ", "x'd", "A", "!", "\n", "ab"]
    docs = []
    for i in range(60):
        k = rng.choice(kinds)
        docs.append(rng.choice(["", "q ", "中"]) + k * rng.randint(0, 3000) + rng.choice(["", " z", "b"]))
    docs += [textgen.cjk_text(300 + i, 2000) for i in range(4)]
    rng.shuffle(docs)
    data, off = textgen.pack_docs(docs)
    want = []
    for d, s in zip(docs, off[:-1]):
        want += [int(s) + p for p in o.pieces(d.encode())]
    same("pieces", gpu_pieces(t, data, off), want)
    ids, out_off = t.encode_batch(data, off)
    want_ids, want_off = oracle_par.concat(oracle_par.map_docs(lambda d: o.encode(d.encode()), docs))
    same("ids", ids, want_ids)
    same("offsets", out_off, want_off)


@pytest.fixture(scope="module")
def walk_back(cfg):
    """The same configuration with no hand-over wait: every tile finds the
    cursor into it by walking back to its segment's cut."""
    merges_name, pattern = libs.CONFIGS["o200k"]
    return tk.Tokenizer(vocab.merges(merges_name), pattern, handoff_wait_us=0)


def test_handoff_wait_range(cfg):
    merges_name, pattern = libs.CONFIGS["o200k"]
    with pytest.raises(tk.TokError) as e:
        tk.Tokenizer(vocab.merges(merges_name), pattern, handoff_wait_us=10_000_001)
    assert e.value.code == tk.TOK_E_ARG


@pytest.mark.parametrize("text", ["A" * 3000 + "b" * 2000 + " x", "中" * 2777 + "A", "7" * 5000 + "x",
                                  " " * 3000 + "y", "x'd" * 1900, "!" + "́" * 2000 + "a", "DON'T" * 600])
def test_walk_back_path(cfg, walk_back, text):
    _, o, _ = cfg
    b = ("pre " + text + " post").encode()
    same("pieces", gpu_pieces(walk_back, b), o.pieces(b))
    same("ids", walk_back.encode(b), o.encode(b))


def test_walk_back_path_workload_and_batch(cfg, walk_back):
    t, o, _ = cfg
    b = textgen.cjk_text(96, 30_000).encode()
    same("pieces", gpu_pieces(walk_back, b), gpu_pieces(t, b))
    docs = random_docs(34, 3000, 40) + ["中" * 1500, "7" * 2100]
    data, off = textgen.pack_docs(docs)
    want = []
    for d, s in zip(docs, off[:-1]):
        want += [int(s) + p for p in o.pieces(d.encode())]
    same("pieces", gpu_pieces(walk_back, data, off), want)
