"""GPU parity of span export (tok_encode_spans, tok_encode_spans_dev): every
token's first byte, next to its ID, against the oracle, which tracks where
each token starts through the merges themselves (TokTier, section 7
"Session-state construction" and Appendix E, "Route C: GPU full tokenization
with span export").  IDs and offsets are integers: the bar is bit-exact.

Covers the workload shapes, ragged sizes around the 1 KiB tile, tiles whose
run holds more tokens than one workgroup pass (long single-character runs
under a tiny vocabulary), documents as hard boundaries with offsets counted
from the start of the concatenated text, capacity overflow, graph replay,
and the 64-document batch workload (sampled documents exactly, all of them by
the property that the spans tile each document with its tokens' lengths).
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


@pytest.fixture(scope="module")
def cfg():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    out = {}
    for name, (merges_name, pattern) in libs.CONFIGS.items():
        m = vocab.merges(merges_name)
        out[name] = (tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern), vocab.token_bytes(m))
    return out


def dev_bytes(b: bytes):
    return torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda() if b else torch.empty(0, dtype=torch.uint8,
                                                                                         device="cuda")


def dev_spans(t, b: bytes, doc_off=None, cap=None):
    d = dev_bytes(b)
    cap = max(len(b), 1) if cap is None else cap
    ids = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    d_off = d_out = None
    if doc_off is not None:
        d_off = torch.tensor(np.asarray(doc_off, dtype=np.int64), device="cuda").view(torch.uint64)
        d_out = torch.zeros(len(doc_off), dtype=torch.int64, device="cuda").view(torch.uint64)
    n = t.encode_spans_dev(d, ids, sp, d_off, d_out)
    torch.cuda.synchronize()
    res = ids[:n].cpu().numpy(), sp[:n].cpu().numpy().view(np.uint32).astype(np.uint64)
    if doc_off is not None:
        return res + (d_out.view(torch.int64).cpu().numpy().astype(np.uint64),)
    return res


def same(what, got, want):
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape or not np.array_equal(got, want):
        n = min(len(got), len(want))
        i = next((k for k in range(n) if got[k] != want[k]), n)
        pytest.fail(f"{what}: {len(got)} vs {len(want)} entries, first difference at {i}: "
                    f"gpu {got[i:i + 5].tolist()} oracle {want[i:i + 5].tolist()}")


@pytest.mark.parametrize("name,gen,seed,n_chars", [
    ("tiny", "tiny", 1, 10_000),
    ("gpt2", "mix", 2, 1_000_000),
    ("llama3", "mix", 3, 3_000_000),
])
def test_workload_spans(cfg, name, gen, seed, n_chars):
    t, o, _ = cfg[name]
    s = textgen.tiny_text(seed, n_chars) if gen == "tiny" else textgen.mix_text(seed, n_chars)
    b = s.encode()
    want_ids, want_sp = o.encode_spans(b)
    ids, sp = t.encode_spans(b)
    same(f"{name} ids", ids, want_ids)
    same(f"{name} spans", sp.astype(np.uint64), want_sp)
    ids, sp = dev_spans(t, b)
    same(f"{name} dev ids", ids, want_ids)
    same(f"{name} dev spans", sp, want_sp)
    # the plain encode is unchanged by the span variant sharing its buffers
    same(f"{name} plain", t.encode(b), want_ids)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_ragged_and_long_runs(cfg, name):
    t, o, _ = cfg[name]
    base = textgen.mix_text(55, 20_000).encode()
    cases = []
    for n in [1, 2, 15, 16, 17, 1023, 1024, 1025, 2049, 4097, 20_000]:
        b = base[:n]
        while b:
            try:
                b.decode()
                break
            except UnicodeDecodeError:
                b = b[:-1]
        cases.append(b)
    rng = random.Random(3)
    cases += [("x" + "1" * 9000 + " " * 7000 + "y").encode(), ("é" * 3000 + "中" * 2000).encode(),
              "".join(rng.choice(["ab", " ", "\n", "12", "'s", "!", "😀"]) for _ in range(6000)).encode()]
    for b in cases:
        want_ids, want_sp = o.encode_spans(b)
        ids, sp = dev_spans(t, b)
        same(f"{name}[{len(b)}] ids", ids, want_ids)
        same(f"{name}[{len(b)}] spans", sp, want_sp)


def test_tile_runs_longer_than_a_pass(cfg):
    """Under the 1,000-merge vocabulary a 10,000-character run of one rare
    character yields thousands of tokens in the run of the tile where the
    piece starts: the span scan carries across many workgroup passes."""
    t, o, _ = cfg["tiny"]
    for s in ["Q" * 10_000, "z" + "é" * 6000 + " x", "(" * 5000 + ")" * 5000, " " * 12_000 + "w"]:
        b = s.encode()
        want_ids, want_sp = o.encode_spans(b)
        ids, sp = dev_spans(t, b)
        same(f"{s[:3]!r} ids", ids, want_ids)
        same(f"{s[:3]!r} spans", sp, want_sp)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_batch_spans(cfg, name):
    t, o, _ = cfg[name]
    docs = ["", "abc 123", "12", "345", "it'", "s fine", "tail   ", "\n  x", "", "中文", "😀😀", "",
            "x" + "9" * 5000, "  \n", "'S", " ", "a" * 300]
    docs += [textgen.mix_text(600 + i, 7000 + 913 * i) for i in range(5)] + [""]
    data, off = textgen.pack_docs(docs)
    want_ids, want_sp, want_off = o.encode_batch_spans(data, off)
    ids, sp, out_off = dev_spans(t, data, off)
    same(f"{name} batch out_off", out_off, want_off)
    same(f"{name} batch ids", ids, want_ids)
    same(f"{name} batch spans", sp, want_sp)


def test_capacity_overflow(cfg):
    t, o, _ = cfg["gpt2"]
    b = textgen.mix_text(8, 30_000).encode()
    want_ids, want_sp = o.encode_spans(b)
    cap = len(want_ids) // 2
    d = dev_bytes(b)
    ids = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(tk.TokError) as e:
        t.encode_spans_dev(d, ids, sp)
    assert e.value.code == tk.TOK_E_CAPACITY
    torch.cuda.synchronize()
    same("first cap ids", ids.cpu().numpy(), want_ids[:cap])
    same("first cap spans", sp.cpu().numpy().view(np.uint32).astype(np.uint64), want_sp[:cap])


def test_graph_replay_with_spans(cfg):
    t, o, _ = cfg["llama3"]
    b = textgen.mix_text(77, 200_000).encode()
    want_ids, want_sp = o.encode_spans(b)
    d = dev_bytes(b)
    ids = torch.empty(len(b), dtype=torch.int32, device="cuda")
    sp = torch.empty(len(b), dtype=torch.int32, device="cuda")
    t.set_graph(True)
    try:
        for k in range(4):
            ids.fill_(-1)
            sp.fill_(-1)
            n = t.encode_spans_dev(d, ids, sp)
            torch.cuda.synchronize()
            same(f"replay {k} ids", ids[:n].cpu().numpy(), want_ids)
            same(f"replay {k} spans", sp[:n].cpu().numpy().view(np.uint32).astype(np.uint64), want_sp)
        assert t.graph_count() >= 1
    finally:
        t.set_graph(False)


def test_batch_workload_spans(cfg):
    """64 documents of 500,000 characters: every document's IDs and spans
    equal the oracle's (spans counted from the batch's first byte), and in
    every document the spans start at its first byte and step by the token
    lengths up to its last byte."""
    t, o, tokb = cfg["llama3"]
    texts = textgen.batch_texts(40_000, 64, 500_000)
    data, off = textgen.pack_docs(texts)
    ids, sp, out_off = dev_spans(t, data, off)
    lens = np.asarray([len(x) for x in tokb], dtype=np.uint64)[ids]
    for i in range(64):
        a, z = int(out_off[i]), int(out_off[i + 1])
        assert sp[a] == off[i]
        assert np.array_equal(sp[a + 1:z], sp[a:z - 1] + lens[a:z - 1])
        assert sp[z - 1] + lens[z - 1] == off[i + 1]
    docs = [data[int(off[i]):int(off[i + 1])] for i in range(64)]
    want = oracle_par.map_docs(o.encode_spans, docs)
    want_ids, want_off = oracle_par.concat([w[0] for w in want])
    same("output offsets", out_off, want_off)
    for i in range(64):
        a, z = int(out_off[i]), int(out_off[i + 1])
        same(f"doc {i} ids", ids[a:z], want[i][0])
        same(f"doc {i} spans", sp[a:z], want[i][1] + np.uint64(off[i]))


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_long_pieces_spans(cfg, name):
    """Spans of pieces over 64 bytes (the long-piece kernel's tokens), single
    request and batch, with documents starting at a long piece: equal to the
    oracle's merge-tracked spans."""
    t, o, _ = cfg[name]
    rng = random.Random(5)
    cjk = lambda k: "".join(chr(rng.randint(0x4E00, 0x9FFF)) for _ in range(k))  # noqa: E731
    docs = [" " * 300 + "x", cjk(500) + ", " + cjk(66), "ab" * 2049, "w" * 65 + " " + cjk(1400), "é" * 80]
    b = "".join(docs).encode()
    ids, sp = dev_spans(t, b)
    want_ids, want_sp = o.encode_spans(b)
    same("single ids", ids, want_ids)
    same("single spans", sp, want_sp)
    data, off = textgen.pack_docs(docs)
    ids, sp, out_off = dev_spans(t, data, off)
    want_ids, want_sp, want_off = o.encode_batch_spans(data, off)
    same("batch ids", ids, want_ids)
    same("batch spans", sp, want_sp)
    same("batch offsets", out_off, want_off)
