"""Append repair over a session kept in device memory (tok_repair_dev): the
match and splice run in one workgroup on the device.  The result must equal
the oracle's full encode of the whole text, and every decision (kept IDs,
splice byte, window start, widenings, fallback) must equal the host repair's
(tok_repair), which runs the same rules on the host.  The stored IDs handed
in are the oracle's encode of the stored text.

Covers the session-append workload (1,000,000-character context, seeded
log-normal appends, 30% starting mid-word or mid-whitespace), seam shapes of
both families, widening and the full-encode fallback, stored IDs that do not
spell the text or do not cover it, capacity overflow (session untouched), an
empty session, added-token literals, and appends of 60K to 1.2M characters
(the long tail copied by a grid-wide kernel), with and without room.
"""
import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEAMS = [
    ("The staging pipe", "line holds"),
    ("one two three\n   ", "\n   four"),
    ("x = 1;\n    ", "    y = 2"),
    ("it'", "s fine and they'll go"),
    ("it", "'s fine"),
    ("count 12345", "6789 items"),
    ("done.\r", "\n\nnext"),
    ("tail   ", "   more"),
    ("emoji \U0001F600", "\U0001F600 and more"),
    ("end", ""),
]


@pytest.fixture(scope="module")
def cfg():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    out = {}
    for name in ("gpt2", "llama3"):
        merges_name, pattern = libs.CONFIGS[name]
        m = vocab.merges(merges_name)
        out[name] = (tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern))
    return out


def dev_repair(t, sess, text: bytes, old_len: int, cap=None):
    sess = np.asarray(sess, dtype=np.int32)
    cap = len(sess) + (len(text) - old_len) + 64 if cap is None else cap
    buf = torch.full((max(cap, 1),), -5, dtype=torch.int32)
    buf[: len(sess)] = torch.from_numpy(sess)
    d = buf.cuda()
    torch.cuda.synchronize()
    n, info = t.repair_dev(d, len(sess), text, old_len)
    return d.cpu().numpy()[:n], info, d


def check(t, o, old: bytes, app: bytes, what: str):
    sess = o.encode(old)
    want = o.encode(old + app)
    got, info, _ = dev_repair(t, sess, old + app, len(old))
    assert np.array_equal(got, want), f"{what}: device repair differs from the full encode ({info})"
    h_ids, h_info = t.repair(sess, old + app, len(old))
    assert h_info == info, f"{what}: device {info} vs host {h_info}"
    if info["full"] == 0:
        assert np.array_equal(got[: info["kept"]], np.asarray(sess)[: info["kept"]])
    return info


def test_session_append_workload(cfg):
    t, o = cfg["gpt2"]
    base = textgen.mix_text(500, 1_000_000)
    full = 0
    for seed in range(24):
        old, suf = textgen.repair_case(500, 9_000 + seed, old_text=base)
        info = check(t, o, old.encode(), suf.encode(), f"append seed {seed}")
        full += info["full"]
    assert full == 0


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_seam_shapes(cfg, name):
    t, o = cfg[name]
    ctx = textgen.mix_text(501, 4_000)
    for left, right in SEAMS:
        check(t, o, (ctx + left).encode(), right.encode(), f"{left!r}|{right!r}")
        check(t, o, left.encode(), right.encode(), f"short {left!r}|{right!r}")


def test_llama3_appends(cfg):
    t, o = cfg["llama3"]
    base = textgen.mix_text(510, 200_000)
    for seed in range(10):
        old, suf = textgen.repair_case(510, 9_500 + seed, old_text=base)
        check(t, o, old.encode(), suf.encode(), f"llama3 append {seed}")


def test_widening_and_fallback(cfg):
    t, o = cfg["gpt2"]
    ctx = textgen.mix_text(502, 3_000)
    info = check(t, o, (ctx + " " + "a" * 3_000).encode(), b"b and c", "widen")
    assert info["full"] == 0 and info["widenings"] >= 3
    info = check(t, o, (ctx + " " + "a" * 20_000).encode(), b"b", "fallback")
    assert info["full"] == 1


def test_session_errors_leave_the_session_alone(cfg):
    t, o = cfg["gpt2"]
    old = textgen.mix_text(503, 5_000).encode()
    app = b" appended words"
    sess = np.asarray(o.encode(old), dtype=np.int32)
    bad = sess.copy()
    bad[-1] = (bad[-1] + 1) % t.info()["vocab_size"]
    for ids in (bad, sess[:-3], np.concatenate([sess[:-1], [t.info()["vocab_size"] + 5]]).astype(np.int32)):
        with pytest.raises(tk.TokError) as e:
            dev_repair(t, ids, old + app, len(old))
        assert e.value.code == tk.TOK_E_SESSION
    # capacity: reported, session untouched
    app = textgen.prose_text(505, 600).encode()
    cap = len(sess)
    buf = torch.from_numpy(sess.copy()).cuda()
    with pytest.raises(tk.TokError) as e:
        t.repair_dev(buf, len(sess), old + app, len(old))
    assert e.value.code == tk.TOK_E_CAPACITY
    assert np.array_equal(buf.cpu().numpy(), sess)
    assert cap == buf.numel()


@pytest.mark.parametrize("with_literals", [False, True])
def test_malformed_append_leaves_the_session_alone(cfg, with_literals):
    """Malformed UTF-8 in the appended bytes, after a stored text cut mid-word:
    the window encode reports it, the match kernel writes nothing, and the
    call returns TOK_E_UTF8 with the device session bit-identical (the window
    IDs after a mid-word cut would otherwise overwrite the stored tail)."""
    t, o = cfg["gpt2"]
    v = t.info()["vocab_size"]
    lits = [(b"<|endoftext|>", v)]
    if with_literals:
        t.set_added_tokens(lits)
    try:
        old = (textgen.mix_text(511, 20_000) + " the wor").encode()
        sess = np.asarray(o.encode_added(old, lits) if with_literals else o.encode(old), dtype=np.int32)
        for app in (b"ld\xff", b"ld and more \xc3", b"ld \xed\xa0\x80 x"):
            buf = torch.from_numpy(np.concatenate([sess, np.full(64, -7, dtype=np.int32)])).cuda()
            with pytest.raises(tk.TokError) as e:
                t.repair_dev(buf, len(sess), old + app, len(old))
            assert e.value.code == tk.TOK_E_UTF8, app
            torch.cuda.synchronize()
            got = buf.cpu().numpy()
            assert np.array_equal(got[:len(sess)], sess) and np.all(got[len(sess):] == -7), app
    finally:
        if with_literals:
            t.set_added_tokens([])


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_empty_session_and_literals(cfg, name):
    t, o = cfg[name]
    app = "Fresh session text, 42 words.\n".encode()
    got, info, _ = dev_repair(t, [], app, 0)
    assert np.array_equal(got, o.encode(app)) and info["full"] == 1
    v = t.info()["vocab_size"]
    lits = [(b"<|endoftext|>", v), (b"<|im_end|>", v + 1)]
    t.set_added_tokens(lits)
    try:
        old = (textgen.mix_text(506, 3000) + "<|im_end|>").encode()
        new = old + b"<|endoftext|> more"
        sess = o.encode_added(old, lits)
        got, info, _ = dev_repair(t, sess, new, len(old))
        assert np.array_equal(got, o.encode_added(new, lits))
        assert t.repair(sess, new, len(old))[1] == info  # the host repair decides the same
    finally:
        t.set_added_tokens([])


@pytest.mark.parametrize("app_chars", [60_000, 250_000, 1_200_000])
def test_large_appends(cfg, app_chars):
    """Appends of 50K characters and more (where TokTier's delta-aware routing
    would re-encode the whole request): the window repair still runs, and its
    result and decisions match the host repair and the full encode, also for
    an append longer than the stored context."""
    t, o = cfg["gpt2"]
    old = textgen.mix_text(520, 300_000)
    app = textgen.mix_text(521 + app_chars, app_chars)
    for cut in (0, 7):  # append starting at a block edge, and mid-word
        info = check(t, o, (old + app[:cut]).encode(), app[cut:].encode(), f"append {app_chars} cut {cut}")
        assert info["full"] == 0


def test_large_append_capacity_and_repeat(cfg):
    """A long tail (copied by the grid-wide kernel) that does not fit the
    session buffer is reported with the required count and leaves the
    session untouched; the same append then fits a larger buffer, and a short
    append after it (inline copy) still matches the full encode."""
    t, o = cfg["gpt2"]
    old = textgen.mix_text(530, 100_000).encode()
    app = textgen.mix_text(531, 120_000).encode()
    sess = np.asarray(o.encode(old), dtype=np.int32)
    want = o.encode(old + app)
    pad = np.full(64, -9, dtype=np.int32)
    buf = torch.from_numpy(np.concatenate([sess, pad])).cuda()
    with pytest.raises(tk.TokError) as e:
        t.repair_dev(buf, len(sess), old + app, len(old))
    assert e.value.code == tk.TOK_E_CAPACITY
    assert np.array_equal(buf.cpu().numpy(), np.concatenate([sess, pad]))
    big = torch.full((len(want) + 16,), -9, dtype=torch.int32)
    big[: len(sess)] = torch.from_numpy(sess)
    d = big.cuda()
    n, info = t.repair_dev(d, len(sess), old + app, len(old))
    assert n == len(want) and info["full"] == 0
    assert np.array_equal(d.cpu().numpy()[:n], want)
    more = b" and a short tail"
    want2 = o.encode(old + app + more)
    d2 = torch.full((len(want2) + 16,), -9, dtype=torch.int32)
    d2[:n] = d[:n].cpu()
    d2 = d2.cuda()
    n2, _ = t.repair_dev(d2, n, old + app + more, len(old + app))
    assert np.array_equal(d2.cpu().numpy()[:n2], want2)
