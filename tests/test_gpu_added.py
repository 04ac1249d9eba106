"""GPU parity of the added-token literal pass (tok_set_added_tokens, then
tok_encode / tok_encode_dev) against the oracle's literal pass, bit-exact.

Covers chat-transcript text with marker literals on both pattern families at
the 1M-character size, literals that also occur inside ordinary code (many
matches per tile), overlapping literal sets (the selection's ordered path),
literals at the text's ends, back to back and across 1 KiB tiles, a 64-byte
literal, one-byte and multibyte literals, text without any occurrence,
capacity overflow, malformed UTF-8, invalid literal sets, removal, batches
(literals within each document, never across a boundary; per-document
offsets; spans), span export with literals (token starts tile the text:
the running sum of the token byte lengths, a literal counting its own
length), and the hand-worked cases of
tests/golden/added_tokens.json (tiny merge tables, run last).
"""
import json
import os
import random

import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, oracle_par, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HERE = os.path.dirname(os.path.abspath(__file__))
MARKERS = ["<|im_start|>", "<|im_end|>", "<|endoftext|>", "<|tool_call|>", "<|im_sep|>"]


@pytest.fixture(scope="module")
def cfg():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    out = {}
    for name, (merges_name, pattern) in libs.CONFIGS.items():
        m = vocab.merges(merges_name)
        out[name] = (tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern), len(m) + 256)
    return out


def lits_from(strings, base):
    return [(s.encode() if isinstance(s, str) else s, base + i) for i, s in enumerate(strings)]


def dev_encode(t, b: bytes, cap=None):
    d = torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda() if b else torch.empty(0, dtype=torch.uint8,
                                                                                     device="cuda")
    ids = torch.full((max(len(b), 1) if cap is None else cap,), -7, dtype=torch.int32, device="cuda")
    n = t.encode_dev(d, ids)
    torch.cuda.synchronize()
    return ids[:n].cpu().numpy()


def same(what, got, want):
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape or not np.array_equal(got, want):
        n = min(len(got), len(want))
        i = next((k for k in range(n) if got[k] != want[k]), n)
        pytest.fail(f"{what}: {len(got)} vs {len(want)} IDs, first difference at {i}: "
                    f"gpu {got[i:i + 6].tolist()} oracle {want[i:i + 6].tolist()}")


def check(t, o, b, lits, what):
    want = o.encode_added(b, lits)
    same(f"{what} host", t.encode(b), want)
    same(f"{what} dev", dev_encode(t, b), want)
    return want


@pytest.mark.parametrize("name,seed,n_chars", [("gpt2", 7, 1_000_000), ("llama3", 8, 1_000_000),
                                               ("tiny", 9, 20_000)])
def test_chat_workload(cfg, name, seed, n_chars):
    t, o, v = cfg[name]
    lits = lits_from(MARKERS, v)
    b = textgen.chat_text(seed, n_chars, MARKERS).encode()
    t.set_added_tokens(lits)
    try:
        want = check(t, o, b, lits, name)
        assert sum(1 for i in want if i >= v) > n_chars // 2000
    finally:
        t.set_added_tokens([])
    same(f"{name} cleared", t.encode(b), o.encode(b))


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_literals_inside_code(cfg, name):
    """Literals that the code blocks contain all the time (operators, a
    keyword, a multibyte letter): thousands of matches, many per tile."""
    t, o, v = cfg[name]
    lits = lits_from(["=>", "==", "return", "->", "é", "self.", "\n    "], v)
    b = textgen.mix_text(17, 300_000).encode()
    t.set_added_tokens(lits)
    try:
        check(t, o, b, lits, name)
    finally:
        t.set_added_tokens([])


def test_overlapping_literals(cfg):
    t, o, v = cfg["gpt2"]
    rng = random.Random(5)
    sets = [["ab", "ba", "aba", "bab"], ["aa", "aaa"], ["a b", " b ", "b a"], ["<|", "|>", "<|x|>", "|x"]]
    for strings in sets:
        lits = lits_from(strings, v)
        t.set_added_tokens(lits)
        try:
            alpha = sorted(set("".join(strings))) + ["x", "\n"]
            for k in range(3):
                b = "".join(rng.choice(alpha) for _ in range(20_000)).encode()
                check(t, o, b, lits, f"{strings} #{k}")
            # one cluster over 200K bytes and more: every tile after the first lists all
            # its matches and the cursor scan runs over the whole list, on a selection
            # grid of several workgroups
            check(t, o, (strings[0] * 100_000).encode(), lits, f"{strings} run")
        finally:
            t.set_added_tokens([])


# operators and indentation that code text holds everywhere, many of them
# overlapping one another (the selection resolves clusters of overlaps)
CODE_LITERALS = ["==", "===", "!=", "!==", "=>", "->", "::", "  ", "    ", "\n    ", "\n        ", "();"]


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_dense_overlapping_literals_on_code(cfg, name):
    t, o, v = cfg[name]
    lits = lits_from(CODE_LITERALS, v)
    b = textgen.tool_text(19, 1_000_000).encode()
    t.set_added_tokens(lits)
    try:
        want = check(t, o, b, lits, name)
        assert sum(1 for i in want if i >= v) > 20_000
        docs = [textgen.tool_text(200 + i, 30_000 + 777 * i) for i in range(8)] + ["", "===", "a ===  b"]
        data, off = textgen.pack_docs(docs)
        ids, out_off = t.encode_batch(data, off)
        want_ids, want_off = oracle_par.concat(oracle_par.map_docs(lambda d: o.encode_added(d.encode(), lits), docs))
        same(f"{name} batch", ids, want_ids)
        same(f"{name} batch offsets", out_off, want_off)
    finally:
        t.set_added_tokens([])


def test_edges(cfg):
    t, o, v = cfg["llama3"]
    long_lit = "<|" + "x" * 60 + "|>"
    assert len(long_lit) == 64
    strings = ["<|eot|>", "<|e", "§", "中文", "😀", long_lit, "\r\n"]
    lits = lits_from(strings, v)
    filler = textgen.mix_text(3, 5000)
    cases = ["", "<|eot|>", "<|eot|><|eot|>", "<|eot|>abc", "abc<|eot|>", "§§§", "a§b", "中文中文x", "😀 😀",
             long_lit, long_lit[:-1], "x" + long_lit + "y", "it's\r\n\r\n ok", "<|e<|eot|>",
             filler[:1020] + "<|eot|>" + filler[1020:3000],        # a literal across the 1 KiB tile edge
             filler[:1023] + "§" + filler[1023:2100] + long_lit,   # a 2-byte literal at the edge
             filler + "<|eot|>" * 300]
    t.set_added_tokens(lits)
    try:
        for s in cases:
            check(t, o, s.encode(), lits, repr(s[:30]))
        with pytest.raises(tk.TokError) as e:
            t.encode(b"ok <|eot|> \xff")
        assert e.value.code == tk.TOK_E_UTF8
        # capacity: the count comes back, the first cap IDs are right
        b = (filler[:2000] + "<|eot|>").encode()
        want = o.encode_added(b, lits)
        cap = len(want) - 3
        d = torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()
        ids = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
        with pytest.raises(tk.TokError) as e:
            t.encode_dev(d, ids)
        assert e.value.code == tk.TOK_E_CAPACITY
        torch.cuda.synchronize()
        same("first cap IDs", ids.cpu().numpy(), want[:cap])
    finally:
        t.set_added_tokens([])


def test_no_occurrence_and_repair(cfg):
    t, o, v = cfg["gpt2"]
    b = textgen.mix_text(21, 200_000).encode()
    lits = lits_from(["<|endoftext|>"], v)
    t.set_added_tokens(lits)
    try:
        same("no occurrence", dev_encode(t, b), o.encode(b))
        # repair splices with literals too, and equals the literal pass
        old = textgen.mix_text(22, 20_000) + "<|endoftext|>"
        new = old + "<|endoftext|> and more"
        sess = o.encode_added(old.encode(), lits)
        ids, info = t.repair(sess, new.encode(), len(old.encode()))
        assert info["full"] == 0
        same("repair", ids, o.encode_added(new.encode(), lits))
    finally:
        t.set_added_tokens([])
    same("cleared", t.encode(b"a<|endoftext|>"), o.encode(b"a<|endoftext|>"))


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_spans_with_literals(cfg, name):
    t, o, v = cfg[name]
    lits = lits_from(MARKERS + ["§", "=>"], v)
    tokb = vocab.token_bytes(vocab.merges(libs.CONFIGS[name][0]))
    t.set_added_tokens(lits)
    try:
        for seed, n_chars in ((31, 300_000), (32, 5_000)):
            b = textgen.chat_text(seed, n_chars, MARKERS).encode()
            b = b.replace(b" = ", b" => ", 50).replace(b"a", "§".encode(), 30)
            want = o.encode_added(b, lits)
            lit_len = {i: len(x) for x, i in lits}
            lens = np.asarray([lit_len[i] if i >= v else len(tokb[i]) for i in want], dtype=np.uint64)
            want_sp = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.uint64)
            assert int(lens.sum()) == len(b)
            ids, sp = t.encode_spans(b)
            same(f"{name} ids", ids, want)
            same(f"{name} spans", sp.astype(np.uint64), want_sp)
            d = torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()
            d_ids = torch.full((len(b),), -7, dtype=torch.int32, device="cuda")
            d_sp = torch.full((len(b),), -7, dtype=torch.int32, device="cuda")
            n = t.encode_spans_dev(d, d_ids, d_sp)
            torch.cuda.synchronize()
            same(f"{name} dev ids", d_ids[:n].cpu().numpy(), want)
            same(f"{name} dev spans", d_sp[:n].cpu().numpy().view(np.uint32).astype(np.uint64), want_sp)
    finally:
        t.set_added_tokens([])


def test_invalid_literal_sets(cfg):
    t, o, v = cfg["gpt2"]
    for bad, code in [([(b"", 1)], tk.TOK_E_ARG), ([(b"x" * 65, 1)], tk.TOK_E_ARG), ([(b"ab", -1)], tk.TOK_E_ARG),
                      ([(b"ab", 1), (b"ab", 2)], tk.TOK_E_ARG), ([(b"\xff", 1)], tk.TOK_E_UTF8),
                      ([(b"\xe4\xb8", 1)], tk.TOK_E_UTF8), ([(b"\xed\xa0\x80", 1)], tk.TOK_E_UTF8)]:
        with pytest.raises(tk.TokError) as e:
            t.set_added_tokens(bad)
        assert e.value.code == code, bad
    same("nothing set", t.encode(b"ab"), o.encode(b"ab"))


BATCH_DOCS = ["", "a<|im_end|>", "<|im_start|>user\nhi", "", "<|im", "_end|>tail", "x" * 5000 + "<|im_sep|>",
              "<|endoftext|>", "<|endoftext|><|endoftext|>", "§=>§", "no literal here", "", "<|tool_call|>"]


def batch_expect(o, docs, lits, v, tokb):
    ids, spans, out_off = [], [], [0]
    lit_len = {i: len(x) for x, i in lits}
    base = 0
    for dtext in docs:
        b = dtext.encode()
        got = o.encode_added(b, lits).tolist()
        lens = [lit_len[i] if i >= v else len(tokb[i]) for i in got]
        at = base
        for L in lens:
            spans.append(at)
            at += L
        assert at == base + len(b)
        ids += got
        out_off.append(len(ids))
        base += len(b)
    return np.asarray(ids, dtype=np.int32), np.asarray(spans, dtype=np.uint64), np.asarray(out_off, dtype=np.uint64)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_batch_with_literals(cfg, name):
    """Each document gets its own literal pass: "<|im" + "_end|>" in two
    documents is no literal; per-document output offsets and spans as the
    oracle's per-document encode."""
    t, o, v = cfg[name]
    lits = lits_from(MARKERS + ["§", "=>"], v)
    tokb = vocab.token_bytes(vocab.merges(libs.CONFIGS[name][0]))
    docs = BATCH_DOCS + [textgen.chat_text(60 + i, 6000 + 977 * i, MARKERS) for i in range(5)] + [""]
    data, off = textgen.pack_docs(docs)
    want_ids, want_sp, want_off = batch_expect(o, docs, lits, v, tokb)
    t.set_added_tokens(lits)
    try:
        ids, out_off = t.encode_batch(data, off)
        same(f"{name} batch out_off", out_off, want_off)
        same(f"{name} batch ids", ids, want_ids)
        d = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
        d_off = torch.tensor(off.astype(np.int64), device="cuda").view(torch.uint64)
        d_out = torch.zeros(len(off), dtype=torch.int64, device="cuda").view(torch.uint64)
        d_ids = torch.full((len(data),), -7, dtype=torch.int32, device="cuda")
        n = t.encode_batch_dev(d, d_off, d_ids, d_out)
        torch.cuda.synchronize()
        same(f"{name} batch dev ids", d_ids[:n].cpu().numpy(), want_ids)
        same(f"{name} batch dev out_off", d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)
        d_sp = torch.full((len(data),), -7, dtype=torch.int32, device="cuda")
        d_out.zero_()
        n = t.encode_spans_dev(d, d_ids, d_sp, d_off, d_out)
        torch.cuda.synchronize()
        same(f"{name} batch spans ids", d_ids[:n].cpu().numpy(), want_ids)
        same(f"{name} batch spans", d_sp[:n].cpu().numpy().view(np.uint32).astype(np.uint64), want_sp)
        same(f"{name} batch spans out_off", d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)
        # malformed offsets are rejected on the device
        bad = torch.tensor(np.asarray([0, 5, 3, len(data)], dtype=np.int64), device="cuda").view(torch.uint64)
        with pytest.raises(tk.TokError) as e:
            t.encode_batch_dev(d, bad, d_ids, torch.zeros(4, dtype=torch.int64, device="cuda").view(torch.uint64))
        assert e.value.code == tk.TOK_E_ARG
    finally:
        t.set_added_tokens([])


def test_batch_workload_with_literals(cfg):
    """64 chat transcripts of 200,000 characters in one batch call: every
    document's IDs and output offsets equal the oracle's encode with the
    literals; every document's IDs cover its bytes."""
    t, o, v = cfg["llama3"]
    lits = lits_from(MARKERS, v)
    tokb = vocab.token_bytes(vocab.merges(libs.CONFIGS["llama3"][0]))
    docs = [textgen.chat_text(7000 + i, 200_000, MARKERS) for i in range(64)]
    data, off = textgen.pack_docs(docs)
    t.set_added_tokens(lits)
    try:
        ids, out_off = t.encode_batch(data, off)
    finally:
        t.set_added_tokens([])
    lit_len = {i: len(x) for x, i in lits}
    lens = np.asarray([lit_len[i] if i >= v else len(tokb[i]) for i in ids.tolist()], dtype=np.int64)
    doc_bytes = np.add.reduceat(lens, out_off[:-1].astype(np.int64))
    assert np.array_equal(doc_bytes, np.diff(off.astype(np.int64)))
    want = oracle_par.map_docs(lambda d: o.encode_added(d.encode(), lits), docs)
    want_ids, want_off = oracle_par.concat(want)
    same("output offsets", out_off, want_off)
    for i in range(64):
        a, z = int(out_off[i]), int(out_off[i + 1])
        same(f"doc {i}", ids[a:z], want[i])


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_random_batches_with_literals(cfg, name):
    """Seeded random batches: many short documents over an alphabet of
    literal fragments, letters, digits, spaces and newlines, so literals sit
    at document edges, straddle them (and must not match), overlap and touch."""
    t, o, v = cfg[name]
    lits = lits_from(["<|a|>", "<|ab|>", "ab", "|>", "<|", "é"], v)
    tokb = vocab.token_bytes(vocab.merges(libs.CONFIGS[name][0]))
    alpha = ["<|", "a", "b", "|>", "<|a|>", " ", "\n", "1", "é", "x", "'s"]
    rng = random.Random(404)
    t.set_added_tokens(lits)
    try:
        for trial in range(6):
            docs = ["".join(rng.choice(alpha) for _ in range(rng.choice([0, 1, 2, 5, 40, 300])))
                    for _ in range(rng.randint(1, 400))]
            data, off = textgen.pack_docs(docs)
            want_ids, want_sp, want_off = batch_expect(o, docs, lits, v, tokb)
            ids, out_off = t.encode_batch(data, off)
            same(f"trial {trial} out_off", out_off, want_off)
            same(f"trial {trial} ids", ids, want_ids)
    finally:
        t.set_added_tokens([])


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_repair_with_literals(cfg, name):
    """Append repair with literals set: a cut never falls inside a literal
    occurrence, taken or not; the result equals the oracle's literal pass over
    the whole text.  Covers appends that complete a literal cut by the seam,
    that begin or end with one, and overlapping literal strings; the device
    session repair takes the same decisions; literal IDs that name vocabulary
    tokens make both encode the whole text."""
    t, o, v = cfg[name]
    lits = lits_from(MARKERS + ["ab|>", "|>x"], v)
    base = textgen.chat_text(90, 60_000, MARKERS)
    seams = [("<|im_", "end|>\nok"), ("<|im_end|", ">"), ("text ", "<|im_start|>user\n"), ("x<|endoftext|>", " y"),
             ("ab", "|>x tail"), ("<", "|tool_call|>{}"), ("", "plain words only")]
    t.set_added_tokens(lits)
    try:
        spliced = 0
        for left, right in seams:
            old = (base + left).encode()
            new = old + right.encode()
            sess = o.encode_added(old, lits)
            want = o.encode_added(new, lits)
            ids, info = t.repair(sess, new, len(old))
            same(f"{left!r}|{right!r}", ids, want)
            spliced += info["full"] == 0
            d = torch.from_numpy(np.concatenate([sess, np.zeros(len(right) + 64, np.int32)]).astype(np.int32)).cuda()
            n, dinfo = t.repair_dev(d, len(sess), new, len(old))
            same(f"dev {left!r}|{right!r}", d[:n].cpu().numpy(), want)
            assert dinfo == info, (left, right, dinfo, info)
        for seed in range(8):
            old_s, suf = textgen.repair_case(91, 9_100 + seed, old_text=base)
            suf = suf[: len(suf) // 2] + MARKERS[seed % len(MARKERS)] + suf[len(suf) // 2:]
            old, new = old_s.encode(), (old_s + suf).encode()
            ids, info = t.repair(o.encode_added(old, lits), new, len(old))
            same(f"append {seed}", ids, o.encode_added(new, lits))
            spliced += info["full"] == 0
        assert spliced >= 8
        # a literal ID that is also a vocabulary ID: the walk-back cannot tell them apart
        clash = [(b"<|im_end|>", 300)]
        t.set_added_tokens(clash)
        old, new = base.encode(), (base + "<|im_end|> more").encode()
        sess = o.encode_added(old, clash)
        ids, info = t.repair(sess, new, len(old))
        assert info["full"] == 1
        same("clash", ids, o.encode_added(new, clash))
        d = torch.from_numpy(np.concatenate([sess, np.zeros(64, np.int32)]).astype(np.int32)).cuda()
        n, dinfo = t.repair_dev(d, len(sess), new, len(old))
        assert dinfo["full"] == 1
        same("clash dev", d[:n].cpu().numpy(), o.encode_added(new, clash))
    finally:
        t.set_added_tokens([])


@pytest.mark.parametrize("count,lo,hi", [(700, 2, 9), (120, 40, 64), (500, 2, 9)])
def test_large_literal_sets(cfg, count, lo, hi):
    """Large literal sets: 700 short literals, 120 of 40-64 bytes (over 6 KiB
    of literal bytes), 500 short ones, with many sharing their first two
    bytes, on text made of them and of their bytes."""
    t, o, v = cfg["gpt2"]
    rng = random.Random(count * 100 + hi)
    alpha = "abcd =\n"
    strings = set()
    while len(strings) < count:
        strings.add("".join(rng.choice(alpha) for _ in range(rng.randint(lo, hi))))
    strings = sorted(strings)
    lits = lits_from(strings, v)
    t.set_added_tokens(lits)
    try:
        pieces = [rng.choice(strings) if rng.random() < 0.3 else rng.choice(alpha) for _ in range(40_000)]
        check(t, o, "".join(pieces).encode(), lits, f"{count} literals of {lo}-{hi} bytes")
    finally:
        t.set_added_tokens([])


def test_many_documents_with_literals(cfg):
    """More document boundaries than a selection workgroup holds in LDS (3,000
    short documents, about 120 KB: a selection grid of several workgroups):
    IDs, output offsets and spans as the oracle's per-document encode; then
    malformed offsets on the same text are rejected, and the next call is
    right again."""
    t, o, v = cfg["gpt2"]
    lits = lits_from(["<|a|>", "==", "===", "ab", "  "], v)
    tokb = vocab.token_bytes(vocab.merges(libs.CONFIGS["gpt2"][0]))
    alpha = ["<|a|>", "=", "==", "a", "b", " ", "  ", "\n", "x", "1", "é"]
    rng = random.Random(2048)
    docs = ["".join(rng.choice(alpha) for _ in range(rng.choice([0, 1, 3, 20, 40, 60]))) for _ in range(3000)]
    data, off = textgen.pack_docs(docs)
    assert len(data) >= 64 * 1024
    want_ids, want_sp, want_off = batch_expect(o, docs, lits, v, tokb)
    t.set_added_tokens(lits)
    try:
        ids, out_off = t.encode_batch(data, off)
        same("out_off", out_off, want_off)
        same("ids", ids, want_ids)
        d = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
        d_off = torch.tensor(off.astype(np.int64), device="cuda").view(torch.uint64)
        d_out = torch.zeros(len(off), dtype=torch.int64, device="cuda").view(torch.uint64)
        d_ids = torch.full((len(data),), -7, dtype=torch.int32, device="cuda")
        d_sp = torch.full((len(data),), -7, dtype=torch.int32, device="cuda")
        n = t.encode_spans_dev(d, d_ids, d_sp, d_off, d_out)
        torch.cuda.synchronize()
        same("spans ids", d_ids[:n].cpu().numpy(), want_ids)
        same("spans", d_sp[:n].cpu().numpy().view(np.uint32).astype(np.uint64), want_sp)
        same("spans out_off", d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)
        bad = off.astype(np.int64).copy()
        bad[1500], bad[1501] = bad[1501] + 1, bad[1500]
        assert bad[1500] > bad[1501]
        d_bad = torch.tensor(bad, device="cuda").view(torch.uint64)
        with pytest.raises(tk.TokError) as e:
            t.encode_batch_dev(d, d_bad, d_ids, d_out)
        assert e.value.code == tk.TOK_E_ARG
        d_out.zero_()
        d_ids.fill_(-7)
        n = t.encode_batch_dev(d, d_off, d_ids, d_out)
        torch.cuda.synchronize()
        same("ids after the rejected call", d_ids[:n].cpu().numpy(), want_ids)
        same("out_off after the rejected call", d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)
    finally:
        t.set_added_tokens([])


def test_batch_literal_errors_and_capacity(cfg):
    """With literals set: malformed UTF-8 in one document rejects the batch;
    a too-small output reports the full count, fills the per-document offsets
    and writes the first cap IDs."""
    t, o, v = cfg["gpt2"]
    lits = lits_from(MARKERS, v)
    tokb = vocab.token_bytes(vocab.merges(libs.CONFIGS["gpt2"][0]))
    t.set_added_tokens(lits)
    try:
        bad = ["<|im_start|>ok", "fine<|im_end|>"]
        data, off = textgen.pack_docs(bad)
        data = data[:3] + b"\xff" + data[4:]
        with pytest.raises(tk.TokError) as e:
            t.encode_batch(data, off)
        assert e.value.code == tk.TOK_E_UTF8
        docs = [textgen.chat_text(80 + i, 3000, MARKERS) for i in range(4)]
        data, off = textgen.pack_docs(docs)
        want_ids, _, want_off = batch_expect(o, docs, lits, v, tokb)
        cap = len(want_ids) - 10
        d = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
        d_off = torch.tensor(off.astype(np.int64), device="cuda").view(torch.uint64)
        d_out = torch.zeros(len(off), dtype=torch.int64, device="cuda").view(torch.uint64)
        d_ids = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
        with pytest.raises(tk.TokError) as e:
            t.encode_batch_dev(d, d_off, d_ids, d_out)
        assert e.value.code == tk.TOK_E_CAPACITY
        torch.cuda.synchronize()
        same("out_off", d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)
        same("first cap IDs", d_ids.cpu().numpy(), want_ids[:cap])
    finally:
        t.set_added_tokens([])


def test_hand_worked_cases():
    libs.ensure_built()
    cases = json.load(open(os.path.join(HERE, "golden", "added_tokens.json")))["cases"]
    for c in cases:
        m = np.asarray(c["merges"], dtype=np.uint32).reshape(-1, 2)
        t = tk.Tokenizer(m, c["pattern"])
        t.set_added_tokens([(s, i) for s, i in c["literals"]])
        b = c["text"].encode()
        assert t.encode(b).tolist() == c["ids"], c["why"]
        if b:
            assert dev_encode(t, b).tolist() == c["ids"], c["why"]
        t.close()
