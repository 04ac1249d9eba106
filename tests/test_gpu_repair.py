"""Append repair (tok_repair) against the CPU oracle's full encode.

The contract is that repair returns exactly the encode of the stored text
plus the append (TokTier, section 3: a miss in the boundary search costs work,
never a different ID; Appendix A, Theorem A.5).  The stored IDs given to
repair are the oracle's encode of the stored text, and the expected result is
the oracle's encode of the whole text, so nothing here depends on the HIP
path's own output.

Covers the session-append workload (a 1,000,000-character context with
log-normal appends, 30% of which start mid-word or mid-whitespace), seam
shapes of both pattern families, window widening and the full-encode
fallback, and rejection of stored IDs that do not spell the stored text.
"""
import ctypes

import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def _repair_check(t, o, old: bytes, app: bytes, what: str):
    sess = o.encode(old)
    got, info = t.repair(sess, old + app, len(old))
    want = o.encode(old + app)
    assert np.array_equal(got, want), f"{what}: repair differs from the full encode ({info})"
    if info["full"] == 0:
        # the kept prefix is untouched stored IDs
        assert np.array_equal(got[: info["kept"]], np.asarray(sess)[: info["kept"]])
    return info


def test_session_append_workload(cfg):
    """1,000,000-char stored context, 24 seeded appends (median 1,400 chars)."""
    t, o = cfg["gpt2"]
    base = textgen.mix_text(500, 1_000_000)
    full = 0
    for seed in range(24):
        old, suf = textgen.repair_case(500, 9_000 + seed, old_text=base)
        info = _repair_check(t, o, old.encode(), suf.encode(), f"append seed {seed}")
        full += info["full"]
        if info["full"] == 0:
            assert info["window_start"] > 0 and info["kept"] > 0
    assert full == 0, "ordinary appends should splice, not re-encode everything"


SEAMS = [
    ("The staging pipe", "line holds"),          # a word cut in the middle
    ("one two three\n   ", "\n   four"),         # newline plus spaces on both sides
    ("x = 1;\n    ", "    y = 2"),               # indentation continued
    ("it'", "s fine and they'll go"),            # contraction across the seam
    ("it", "'s fine"),
    ("count 12345", "6789 items"),               # digit groups shift (Llama-3 style)
    ("done.\r", "\n\nnext"),                      # CR/LF after other chars
    ("tail   ", "   more"),                       # whitespace run continued
    ("emoji \U0001F600", "\U0001F600 and more"),
    ("end", ""),                                  # nothing appended
]


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_seam_shapes(cfg, name):
    t, o = cfg[name]
    ctx = textgen.mix_text(501, 4_000)
    for left, right in SEAMS:
        _repair_check(t, o, (ctx + left).encode(), right.encode(), f"{left!r}|{right!r}")
        _repair_check(t, o, left.encode(), right.encode(), f"short {left!r}|{right!r}")


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_empty_session_is_a_full_encode(cfg, name):
    t, o = cfg[name]
    app = "Fresh session text, 42 words.\n".encode()
    got, info = t.repair([], app, 0)
    assert np.array_equal(got, o.encode(app)) and info["full"] == 1


def test_window_widens_then_falls_back(cfg):
    t, o = cfg["gpt2"]
    ctx = textgen.mix_text(502, 3_000)
    # no class change in the last 3,000 code points: the window must reach 4,096
    info = _repair_check(t, o, (ctx + " " + "a" * 3_000).encode(), "b and c".encode(), "widen")
    assert info["full"] == 0 and info["widenings"] >= 3
    # no class change within the widest window: the whole text is encoded
    info = _repair_check(t, o, (ctx + " " + "a" * 20_000).encode(), "b".encode(), "fallback")
    assert info["full"] == 1


def _raw_repair(t, sess, text: bytes, old_len: int, cap: int):
    buf = np.zeros(max(cap, 1), dtype=np.int32)
    buf[: len(sess)] = sess
    n = ctypes.c_size_t(0)
    info = tk.RepairInfo()
    rc = tk.lib().tok_repair(t._h, buf.ctypes.data, len(sess), cap, text, old_len, len(text), ctypes.byref(n),
                             ctypes.byref(info))
    return rc, n.value, buf


def test_rejects_stored_ids_that_do_not_spell_the_text(cfg):
    t, o = cfg["gpt2"]
    old = textgen.mix_text(503, 5_000).encode()
    app = " appended words".encode()
    sess = np.asarray(o.encode(old), dtype=np.int32)
    bad = sess.copy()
    bad[-1] = (bad[-1] + 1) % t.info()["vocab_size"]
    rc, _, _ = _raw_repair(t, bad, old + app, len(old), len(sess) + len(app))
    assert rc == tk.TOK_E_SESSION
    rc, _, _ = _raw_repair(t, sess[:-3], old + app, len(old), len(sess) + len(app))
    assert rc == tk.TOK_E_SESSION
    rc, _, _ = _raw_repair(t, sess, old + app, len(old) + len(app) + 1, len(sess) + len(app))
    assert rc == tk.TOK_E_ARG


def test_capacity_is_reported_and_ids_untouched(cfg):
    t, o = cfg["gpt2"]
    old = textgen.mix_text(504, 5_000).encode()
    app = textgen.prose_text(505, 600).encode()
    sess = np.asarray(o.encode(old), dtype=np.int32)
    rc, need, buf = _raw_repair(t, sess, old + app, len(old), len(sess))
    assert rc == tk.TOK_E_CAPACITY
    assert need == len(o.encode(old + app))
    assert np.array_equal(buf[: len(sess)], sess)


@pytest.mark.parametrize("opts", [
    dict(repair_window=16, repair_doublings=0, repair_margin=0),
    dict(repair_window=64, repair_doublings=2, repair_margin=0),
    dict(repair_window=2048, repair_doublings=5, repair_margin=64),
    dict(repair_window=1, repair_doublings=24, repair_margin=1000, initial_bytes=1 << 22),
])
def test_repair_options(cfg, opts):
    """Load options (tok_opts) change only how much work a repair does, never
    its result: every window, doubling count and margin gives the full
    encode, on the host and the device session; the first window and the
    doublings bound where the window starts."""
    merges_name, pattern = libs.CONFIGS["gpt2"]
    t = tk.Tokenizer(vocab.merges(merges_name), pattern, **opts)
    o = cfg["gpt2"][1]
    base = textgen.mix_text(531, 60_000)
    try:
        for seed in range(10):
            old, suf = textgen.repair_case(531, 9_500 + seed, old_text=base)
            ob, text = old.encode(), (old + suf).encode()
            sess = o.encode(ob)
            want = o.encode(text)
            got, info = t.repair(sess, text, len(ob))
            assert np.array_equal(got, want), (seed, info)
            assert info["widenings"] <= opts["repair_doublings"]
            if not info["full"]:
                w = opts["repair_window"] << info["widenings"]
                assert len(old) - len(text[: info["window_start"]].decode()) <= w
            buf = torch.from_numpy(np.concatenate([sess, np.zeros(len(want) + 8, np.int32)])).cuda()
            n, dinfo = t.repair_dev(buf, len(sess), text, len(ob))
            assert dinfo == info and np.array_equal(buf[:n].cpu().numpy(), want)
    finally:
        t.close()
