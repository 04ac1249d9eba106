"""Graph replay (tok_set_graph) against the CPU oracle.

A replayed graph bakes in its launch arguments, so these tests change what
the buffers hold between replays of one shape and check every replay against
the oracle, with the program's own device work and synchronizations in
between (GraphTok, section 6.2: stale state across replays and context
growth).  Also: errors and capacity overflow reported by a replay, batch and
host-memory calls, eviction, growth of the context's buffers, and calls with
stage timing, which run eagerly.
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
def pairs():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    out = {}
    for name in ("gpt2", "llama3", "o200k"):
        merges_name, pattern = libs.CONFIGS[name]
        m = vocab.merges(merges_name)
        out[name] = (tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern))
    return out


@pytest.fixture
def graph_on(pairs):
    for t, _ in pairs.values():
        t.set_graph(True)
    yield pairs
    for t, _ in pairs.values():
        t.set_graph(False)
        assert t.graph_count() == 0


def fixed_len_text(seed: int, n: int) -> bytes:
    """Seeded mixed text cut at a code-point boundary and padded to n bytes."""
    b = textgen.mix_text(seed, n).encode()[:n].decode("utf-8", "ignore").encode()
    return b + b"q" * (n - len(b))


def raw_encode_dev(t, d_text, n, d_ids, cap):
    out = ctypes.c_size_t(0)
    rc = tk.lib().tok_encode_dev(t._h, d_text.data_ptr(), n, d_ids.data_ptr(), cap, ctypes.byref(out), None)
    return rc, out.value


@pytest.mark.parametrize("name", ["gpt2", "llama3", "o200k"])
def test_replay_follows_buffer_contents(graph_on, name):
    t, o = graph_on[name]
    n = 200_000
    texts = [fixed_len_text(700 + i, n) for i in range(6)]
    # all contents on the device; each call's input is a device-to-device copy
    # on torch's current stream, queued right before the call
    src = torch.frombuffer(bytearray(b"".join(texts)), dtype=torch.uint8).cuda()
    d_text = torch.empty(n, dtype=torch.uint8, device="cuda")
    d_ids = torch.empty(n, dtype=torch.int32, device="cuda")
    counts = []
    for rep in range(2):
        for i, b in enumerate(texts):
            d_text.copy_(src[i * n:(i + 1) * n])
            d_ids.fill_(-1)
            k = t.encode_dev(d_text, d_ids)
            counts.append(t.graph_count())
            got = d_ids[:k].cpu().numpy()
            torch.cuda.synchronize()
            want = o.encode(b)
            assert np.array_equal(got, want), f"replay {rep}/{i} differs from the oracle"
            assert np.all(d_ids[k:].cpu().numpy() == -1), "wrote past the count"
    assert counts[0] == 0 and all(c == 1 for c in counts[1:]), counts


def stretch_text(seed: int, n: int) -> bytes:
    """Mixed text of n bytes with stretches that hold no synchronizing cut of
    the case-splitting family (digits, spaces, contractions, an ideograph
    run) placed by the seed, so that the cursors the tiles hand over differ
    from text to text."""
    rng = np.random.default_rng(seed)
    parts, size = [], 0
    while size < n:
        k = int(rng.integers(0, 5))
        if k == 0:
            s = textgen.mix_text(int(rng.integers(1 << 30)), int(rng.integers(200, 3000)))
        elif k == 1:
            s = " 7" + "7" * int(rng.integers(1000, 6000))
        elif k == 2:
            s = "x" + " " * int(rng.integers(1000, 5000)) + "y"
        elif k == 3:
            s = " " + "x'd" * int(rng.integers(300, 2000))
        else:
            s = "，" + "中" * int(rng.integers(200, 400)) + "。"
        parts.append(s)
        size += len(s.encode())
    return fixed_len_text_from("".join(parts).encode(), n)


def fixed_len_text_from(b: bytes, n: int) -> bytes:
    b = b[:n].decode("utf-8", "ignore").encode()
    return b + b"q" * (n - len(b))


def test_replay_hands_over_fresh_cursors(graph_on):
    """Under the case-splitting family each tile takes the cursor its
    predecessor publishes in the call; a replay bakes in the call number it
    was captured with, so the words must be told apart by a number the
    device advances itself.  Texts with cut-free stretches in different
    places, replayed twice each, against the oracle."""
    t, o = graph_on["o200k"]
    n = 150_000
    texts = [stretch_text(900 + i, n) for i in range(5)]
    src = torch.frombuffer(bytearray(b"".join(texts)), dtype=torch.uint8).cuda()
    d_text = torch.empty(n, dtype=torch.uint8, device="cuda")
    d_ids = torch.empty(n, dtype=torch.int32, device="cuda")
    wants = [o.encode(b) for b in texts]
    for rep in range(2):
        for i in range(len(texts)):
            d_text.copy_(src[i * n:(i + 1) * n])
            k = t.encode_dev(d_text, d_ids)
            assert np.array_equal(d_ids[:k].cpu().numpy(), wants[i]), f"replay {rep}/{i} differs from the oracle"
    assert t.graph_count() == 1


def test_replay_reports_errors_and_capacity(graph_on):
    t, o = graph_on["gpt2"]
    n = 50_000
    good = fixed_len_text(710, n)
    bad = bytearray(good)
    bad[n // 2] = 0xFF
    d_text = torch.empty(n, dtype=torch.uint8, device="cuda")
    want = o.encode(good)
    cap = len(want)
    d_ids = torch.empty(cap, dtype=torch.int32, device="cuda")
    # dense digits need more tokens than cap for the same shape
    many = (b"7 " * (n // 2))[:n]
    many_want = o.encode(many)
    assert len(many_want) > cap
    for rep in range(3):
        d_text.copy_(torch.frombuffer(bytearray(good), dtype=torch.uint8))
        rc, k = raw_encode_dev(t, d_text, n, d_ids, cap)
        assert rc == tk.TOK_OK and k == cap
        assert np.array_equal(d_ids.cpu().numpy(), want)
        d_text.copy_(torch.frombuffer(bad, dtype=torch.uint8))
        rc, k = raw_encode_dev(t, d_text, n, d_ids, cap)
        assert rc == tk.TOK_E_UTF8 and k == 0, (rep, rc, k)
        d_text.copy_(torch.frombuffer(bytearray(many), dtype=torch.uint8))
        rc, k = raw_encode_dev(t, d_text, n, d_ids, cap)
        assert rc == tk.TOK_E_CAPACITY and k == len(many_want), (rep, rc, k)
        assert np.array_equal(d_ids.cpu().numpy(), many_want[:cap])
    assert t.graph_count() == 1


def test_batch_replay(graph_on):
    t, o = graph_on["llama3"]
    n_docs, total = 16, 120_000
    rng = np.random.default_rng(5)
    d_text = torch.empty(total, dtype=torch.uint8, device="cuda")
    d_doc = torch.empty(n_docs + 1, dtype=torch.int64, device="cuda")
    d_ids = torch.empty(total, dtype=torch.int32, device="cuda")
    d_out = torch.empty(n_docs + 1, dtype=torch.int64, device="cuda")
    for rep in range(4):
        data = fixed_len_text(720 + rep, total)
        # cuts at code-point starts, including empty documents
        starts = [i for i in range(total) if data[i] & 0xC0 != 0x80]
        cuts = np.sort(rng.choice(starts, n_docs - 1, replace=True))
        off = np.concatenate([[0], cuts, [total]]).astype(np.uint64)
        d_text.copy_(torch.frombuffer(bytearray(data), dtype=torch.uint8))
        d_doc.copy_(torch.from_numpy(off.astype(np.int64)))
        k = t.encode_batch_dev(d_text, d_doc.view(torch.uint64), d_ids, d_out.view(torch.uint64))
        want_ids, want_off = o.encode_batch(data, off)
        assert np.array_equal(d_out.cpu().numpy().astype(np.uint64), want_off), rep
        assert np.array_equal(d_ids[:k].cpu().numpy(), want_ids), rep
    assert t.graph_count() == 1


def test_host_path_replay_and_growth(graph_on):
    t, o = graph_on["gpt2"]
    for i in range(4):
        b = fixed_len_text(730 + i, 30_000)
        assert np.array_equal(t.encode(b), o.encode(b))
    assert t.graph_count() == 1
    # a request larger than every buffer so far regrows them and drops the graphs
    big = fixed_len_text(740, 9_000_000)
    assert np.array_equal(t.encode(big), o.encode(big))
    assert t.graph_count() == 0
    for i in range(3):
        b = fixed_len_text(750 + i, 30_000)
        assert np.array_equal(t.encode(b), o.encode(b))
    assert t.graph_count() == 1


def test_eviction_keeps_at_most_eight(graph_on):
    t, o = graph_on["gpt2"]
    texts = [fixed_len_text(760 + i, 4_000 + 97 * i) for i in range(11)]
    for rep in range(2):
        for b in texts:
            assert np.array_equal(t.encode(b), o.encode(b))
    assert t.graph_count() == 8
    for b in texts[:3]:  # evicted shapes come back
        assert np.array_equal(t.encode(b), o.encode(b))
    assert t.graph_count() == 8


def test_timed_calls_run_eagerly(graph_on):
    t, o = graph_on["gpt2"]
    b = fixed_len_text(780, 64_000)
    t.set_profiling(True)
    try:
        for _ in range(3):
            assert np.array_equal(t.encode(b), o.encode(b))
            assert t.graph_count() == 0
            assert all(ms > 0 for ms in t.stage_ms())
    finally:
        t.set_profiling(False)
    for _ in range(2):
        assert np.array_equal(t.encode(b), o.encode(b))
    assert t.graph_count() == 1


def test_repair_with_graphs_on(graph_on):
    t, o = graph_on["gpt2"]
    base = textgen.mix_text(790, 200_000)
    for seed in range(6):
        old, suf = textgen.repair_case(790, 9_100 + seed, old_text=base)
        old_b, full_b = old.encode(), (old + suf).encode()
        got, info = t.repair(o.encode(old_b), full_b, len(old_b))
        assert np.array_equal(got, o.encode(full_b)), info


MARKERS = ["<|im_start|>", "<|im_end|>", "<|endoftext|>", "<|tool_call|>", "<|im_sep|>"]


def test_literal_path_replay(graph_on):
    """The literal pass and the pipeline after it captured as one graph: the
    parts' count is read on the device, so replays with other texts of the
    same length (other literal counts) match the oracle; a new literal set
    drops the graphs, and batches replay too."""
    t, o = graph_on["gpt2"]
    v = t.info()["vocab_size"]
    lits = [(m.encode(), v + i) for i, m in enumerate(MARKERS)]
    t.set_added_tokens(lits)
    try:
        n = 120_000
        d_text = torch.empty(n, dtype=torch.uint8, device="cuda")
        d_ids = torch.empty(n, dtype=torch.int32, device="cuda")
        counts = []
        for rep in range(6):
            b = textgen.chat_text(900 + rep, n, MARKERS).encode()[:n].decode("utf-8", "ignore").encode()
            b = b + b" " * (n - len(b))
            d_text.copy_(torch.frombuffer(bytearray(b), dtype=torch.uint8))
            d_ids.fill_(-1)
            k = t.encode_dev(d_text, d_ids)
            counts.append(t.graph_count())
            got = d_ids[:k].cpu().numpy()
            torch.cuda.synchronize()
            assert np.array_equal(got, o.encode_added(b, lits)), f"replay {rep}"
        assert counts[0] == 0 and all(c == 1 for c in counts[1:]), counts
        # a new literal set: no graph survives, and the next shape captures again
        lits2 = lits + [(b"==", v + 7)]
        t.set_added_tokens(lits2)
        assert t.graph_count() == 0
        for rep in range(3):
            b = (textgen.tool_text(950 + rep, n).encode()[:n].decode("utf-8", "ignore").encode())
            b = b + b" " * (n - len(b))
            d_text.copy_(torch.frombuffer(bytearray(b), dtype=torch.uint8))
            k = t.encode_dev(d_text, d_ids)
            assert np.array_equal(d_ids[:k].cpu().numpy(), o.encode_added(b, lits2)), f"after reset {rep}"
        assert t.graph_count() == 1
        # a batch with literals
        docs = [textgen.chat_text(960 + i, 9_000, MARKERS) for i in range(5)]
        data, off = textgen.pack_docs(docs)
        d_b = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
        d_doc = torch.from_numpy(off.astype(np.int64)).cuda().view(torch.uint64)
        d_bid = torch.empty(len(data), dtype=torch.int32, device="cuda")
        d_out = torch.empty(len(docs) + 1, dtype=torch.int64, device="cuda").view(torch.uint64)
        want = [o.encode_added(d.encode(), lits2) for d in docs]
        for rep in range(3):
            k = t.encode_batch_dev(d_b, d_doc, d_bid, d_out)
            assert np.array_equal(d_bid[:k].cpu().numpy(), np.concatenate(want)), f"batch {rep}"
            offs = d_out.view(torch.int64).cpu().numpy()
            assert np.array_equal(np.diff(offs), [len(w) for w in want]), f"batch offsets {rep}"
    finally:
        t.set_added_tokens([])
