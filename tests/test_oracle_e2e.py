"""End-to-end invariants of the oracle and pins of the merge-list trainer.

C-P1 the token byte strings concatenate to the input bytes;
C-P2 0 < T <= N bytes for non-empty input, T = 0 for empty input;
C-P3 determinism;
C-P5 a batch equals its documents encoded one by one (documents are hard
     boundaries: GraphTok, section 5, "Batch entry point").
Trainer: a hand-worked corpus, tie-breaking, unique token strings, and a
re-run that must reproduce the committed artifact bit for bit.
"""
import hashlib
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from synth import textgen
from synth.train_vocab import build_trainer
from tests import vocab


@pytest.fixture(scope="module")
def gpt2():
    m = vocab.merges("gpt2_50k")
    return oracle.Oracle(m, "gpt2"), vocab.token_bytes(m)


@pytest.fixture(scope="module")
def llama():
    m = vocab.merges("llama3_128k")
    return oracle.Oracle(m, "llama3"), vocab.token_bytes(m)


def test_roundtrip_and_counts(gpt2, llama):
    for (o, tok), seed in ((gpt2, 2), (llama, 3)):
        text = textgen.mix_text(seed, 200_000)
        b = text.encode()
        ids = o.encode(b)
        assert vocab.detok(ids, tok) == b
        assert 0 < len(ids) <= len(b)
        assert np.array_equal(ids, o.encode(b))
    assert len(gpt2[0].encode(b"")) == 0


def test_tiny_workload_roundtrip():
    m = vocab.merges("tiny_1k")
    o, tok = oracle.Oracle(m, "gpt2"), vocab.token_bytes(m)
    b = textgen.tiny_text(1).encode()
    assert len(b) == 10_000
    assert vocab.detok(o.encode(b), tok) == b


def test_batch_equals_per_doc(llama):
    o, _ = llama
    docs = ["", "abc 123", "12", "345", "it'", "s fine", "tail   ", "\n  x", "", "中文", "😀😀", ""]
    docs += [textgen.mix_text(400 + i, 3000) for i in range(4)]
    data, off = textgen.pack_docs(docs)
    ids, out_off = o.encode_batch(data, off)
    for d, t in enumerate(docs):
        want = o.encode(t)
        got = ids[int(out_off[d]):int(out_off[d + 1])]
        assert np.array_equal(got, want), d


def test_batch_rejects_bad_utf8(llama):
    o, _ = llama
    data, off = textgen.pack_docs(["ok", "fine"])
    with pytest.raises(UnicodeDecodeError):
        o.encode_batch(b"ok\xe4\xb8", np.array([0, 2, 4], dtype=np.uint64))
    # a character split across two documents is malformed in each
    b = "a中b".encode()
    with pytest.raises(UnicodeDecodeError):
        o.encode_batch(b, np.array([0, 2, len(b)], dtype=np.uint64))


def _train(words: dict, n_merges: int) -> list:
    exe = build_trainer()
    with tempfile.TemporaryDirectory() as d:
        wp, mp = os.path.join(d, "w"), os.path.join(d, "m")
        with open(wp, "wb") as f:
            items = sorted(words.items())
            f.write(struct.pack("<Q", len(items)))
            for k, v in items:
                f.write(struct.pack("<QI", v, len(k)))
                f.write(k)
        r = subprocess.run([exe, wp, str(n_merges), mp], capture_output=True)
        if r.returncode:
            return None
        return np.fromfile(mp, dtype="<u4").reshape(-1, 2).tolist()


def test_trainer_hand_example():
    # counts: ab 3+2=5, bc 2+1=3 -> (a,b) first; then (256,c)=2 beats (b,c)=1; then (b,c)
    assert _train({b"ab": 3, b"abc": 2, b"bc": 1}, 3) == [[97, 98], [256, 99], [98, 99]]
    # equal counts: smallest (left, right) first
    assert _train({b"cd": 1, b"ab": 1}, 2) == [[97, 98], [99, 100]]
    # pairs run out -> error
    assert _train({b"ab": 1}, 2) is None


def test_trainer_reproduces_artifact():
    from synth import train_vocab
    with tempfile.TemporaryDirectory() as d:
        old = train_vocab.VOCAB_DIR
        train_vocab.VOCAB_DIR = d
        try:
            info = train_vocab.train("tiny_1k", workers=1)
        finally:
            train_vocab.VOCAB_DIR = old
    assert info["sha256"] == vocab.MANIFEST["tiny_1k"]["sha256"]


@pytest.mark.parametrize("name", ["tiny_1k", "gpt2_50k", "llama3_128k"])
def test_vocab_strings_unique(name):
    tok = vocab.token_bytes(vocab.merges(name))
    assert len(set(tok)) == len(tok)


def _spans_from_bytes(ids, tok, start=0):
    """Token start bytes as the running sum of the tokens' byte lengths (the
    gather-and-cumulative-sum reading of span export, TokTier, Appendix E,
    "Route C: GPU full tokenization with span export")."""
    lens = np.array([len(tok[i]) for i in ids], dtype=np.uint64)
    return start + np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.uint64) if len(ids) else lens


def test_spans_follow_the_merges(gpt2, llama):
    """The oracle tracks where each token starts through the merges themselves;
    pinned here against the token byte strings: every span slices the text to
    exactly its token's bytes, and the spans are the running sum of lengths."""
    for (o, tok), seed in ((gpt2, 2), (llama, 3)):
        b = textgen.mix_text(seed + 70, 50_000).encode()
        ids, sp = o.encode_spans(b)
        assert np.array_equal(ids, o.encode(b))
        assert np.array_equal(sp, _spans_from_bytes(ids, tok))
        ends = list(sp[1:]) + [len(b)]
        assert all(b[int(s):int(e)] == tok[i] for s, e, i in zip(sp, ends, ids))
    ids, sp = gpt2[0].encode_spans(b"")
    assert len(ids) == 0 and len(sp) == 0


def test_batch_spans_are_absolute(llama):
    """Batch spans count from the start of the concatenated text; every
    document's first token starts at the document's first byte."""
    o, tok = llama
    docs = ["", "abc 123", "中文 x", "", "it's\r\n  ok", textgen.mix_text(91, 2000)]
    data = "".join(docs).encode()
    off = np.cumsum([0] + [len(d.encode()) for d in docs]).astype(np.uint64)
    ids, sp, out_off = o.encode_batch_spans(data, off)
    for d in range(len(docs)):
        a, z = int(out_off[d]), int(out_off[d + 1])
        want_ids = o.encode(docs[d].encode())
        assert np.array_equal(ids[a:z], want_ids)
        assert np.array_equal(sp[a:z], _spans_from_bytes(want_ids, tok, int(off[d])))
