"""GPU parity: the HIP pipeline, called through the C ABI, against the CPU
oracle, element by element.  Token IDs and piece offsets are integers, so the
bar is bit-exact equality everywhere.

Covers the five workload shapes (tiny ASCII, 1M-char request, 3M-char
Llama-3-style request, a 64-document batch, and the seams that append repair
creates), split-level parity of the pre-tokenizer alone (TokTier, section 5.2
compares pieces before IDs), ragged sizes around the 16-byte chunk and 4 KiB
tile, pieces long enough for the long-piece kernel (GraphTok, section 6.2:
long pre-tokens, 10,000-character runs of one character), malformed UTF-8,
capacity overflow, documents as hard boundaries, and stale state across calls
of different sizes on one context (GraphTok, section 6.2: stale state across
replays).
"""
import ctypes
import random

import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, oracle_par, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALPHA = ["a", "b", "s", "t", "r", "e", "l", "d", "S", "ſ", "'", " ", "\n", "\r", "\t", "1", "2",
         "!", ".", " ", "é", "中", "́", "\U0001F600", "\u0085"]


def _pair(name):
    merges_name, pattern = libs.CONFIGS[name]
    m = vocab.merges(merges_name)
    return tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern), vocab.token_bytes(m)


@pytest.fixture(scope="module")
def cfg():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return {name: _pair(name) for name in libs.CONFIGS}


def dev_bytes(b: bytes):
    return torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda() if b else torch.empty(0, dtype=torch.uint8,
                                                                                         device="cuda")


def gpu_pieces(t: tk.Tokenizer, b: bytes, doc_off=None):
    d = dev_bytes(b)
    flags = torch.zeros((len(b) + 15) // 16 + 8, dtype=torch.int16, device="cuda")
    doc = None if doc_off is None else torch.tensor(np.asarray(doc_off, dtype=np.int64), device="cuda").view(
        torch.uint64)
    t.pretokenize_dev(d, flags, doc)
    torch.cuda.synchronize()
    return tk.flags_to_starts(flags.cpu().numpy().view(np.uint16), len(b)).tolist()


def gpu_encode_dev(t: tk.Tokenizer, b: bytes):
    d = dev_bytes(b)
    ids = torch.empty(max(len(b), 1), dtype=torch.int32, device="cuda")
    n = t.encode_dev(d, ids)
    torch.cuda.synchronize()
    return ids[:n].cpu().numpy()


def adversarial_texts():
    rng = random.Random(2024)
    rand = "".join("".join(rng.choice(ALPHA) for _ in range(rng.randint(1, 30))) + rng.choice(ALPHA)
                   for _ in range(8000))
    return [
        rand,
        "x" + "1" * 10001 + "y" + "22" * 3000,        # digit runs across tiles
        "a" + " " * 9000 + "b" + " " * 5000,          # whitespace run across tiles, trailing run
        "q\n" + " " * 6000 + "\n  z" + "\n" * 4097,   # CR/LF far apart inside one run
        "!" + "\r\n" * 5000 + "  w\t\t x",            # CR/LF block after O spanning tiles
        "it's " * 900 + "IT'S 'LL 'Re 'ſ 'x",        # contractions
        "  \u0085 z" * 1500,                     # non-ASCII whitespace
        "中文字" * 3000 + "😀" * 1200,               # multibyte letters and other
    ]


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_split_parity(cfg, name):
    t, o, _ = cfg[name]
    for s in adversarial_texts() + [textgen.mix_text(91, 300_000)]:
        b = s.encode()
        got, want = gpu_pieces(t, b), o.pieces(b)
        if got != want:
            i = next(k for k in range(min(len(got), len(want))) if got[k] != want[k])
            pytest.fail(f"{name}: first split difference at piece {i}: gpu {got[i]} oracle {want[i]}, "
                        f"context {b[max(0, want[i] - 20):want[i] + 20]!r}")


def test_load_info(cfg):
    for name, (t, _, tokb) in cfg.items():
        info = t.info()
        assert info["vocab_size"] == len(tokb)
        assert info["max_token_len"] == max(len(x) for x in tokb)
        # every trained vocabulary string encodes to its own ID (checked by the
        # oracle tests), so the load-time check must admit all 2..28-byte ones
        assert info["n_not_self"] == 0, name
        assert info["n_whole"] == sum(1 for x in tokb[256:] if 2 <= len(x) <= 28)
        assert np.array_equal(t.token_lengths(), [len(x) for x in tokb])


def _check(name, got, want, b, tokb):
    if not np.array_equal(got, want):
        n = min(len(got), len(want))
        i = next((k for k in range(n) if got[k] != want[k]), n)
        pytest.fail(f"{name}: {len(got)} vs {len(want)} tokens, first difference at {i}: "
                    f"gpu {got[i:i + 5].tolist()} oracle {want[i:i + 5].tolist()}")


@pytest.mark.parametrize("name,gen,seed,n_chars", [
    ("tiny", "tiny", 1, 10_000),
    ("gpt2", "mix", 2, 1_000_000),
    ("gpt2", "mix", 21, 2_500_000),   # more tiles than one device generation: 4-wave piece workgroups
    ("llama3", "mix", 3, 3_000_000),
    ("llama3", "mix", 31, 700_000),   # fewer tiles than one generation: 8-wave piece workgroups
])
def test_workload_parity(cfg, name, gen, seed, n_chars):
    t, o, tokb = cfg[name]
    s = textgen.tiny_text(seed, n_chars) if gen == "tiny" else textgen.mix_text(seed, n_chars)
    b = s.encode()
    want = o.encode(b)
    _check(name, t.encode(b), want, b, tokb)
    _check(name, gpu_encode_dev(t, b), want, b, tokb)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_high_id_vocabulary_strings(cfg, name):
    """Text made of the latest merges' strings (IDs from 33,024 on), each a
    piece of its own: whole-piece table hits for nearly all of them, beside
    pieces that are not vocabulary strings (the newlines between), must come
    out as the oracle encodes them."""
    t, o, tokb = cfg[name]
    def utf8(x):
        try:
            x.decode("utf-8")
            return True
        except UnicodeDecodeError:
            return False

    picks = [x for i, x in enumerate(tokb) if i >= 256 + 32768 and 2 <= len(x) <= 28 and utf8(x)]
    whole = [x for x in picks if o.pieces(x) == [0]]
    assert len(whole) > 1000
    b = b"\n".join(whole)
    _check(name, t.encode(b), o.encode(b), b, tokb)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_adversarial_parity(cfg, name):
    t, o, tokb = cfg[name]
    for s in adversarial_texts():
        b = s.encode()
        _check(name, t.encode(b), o.encode(b), b, tokb)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_ragged_sizes(cfg, name):
    t, o, tokb = cfg[name]
    base = textgen.mix_text(5, 40_000).encode()
    for n in [1, 2, 3, 15, 16, 17, 31, 33, 63, 64, 65, 1023, 1024, 1025, 2047, 2048, 4095, 4096, 4097, 4160,
              8191, 8192, 12289, 40_000]:
        b = base[:n]
        while b:
            try:
                b.decode()
                break
            except UnicodeDecodeError:
                b = b[:-1]
        _check(f"{name}[{n}]", t.encode(b), o.encode(b), b, tokb)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
@pytest.mark.parametrize("total", [700_000, 1_600_000])
def test_long_runs_in_large_input(cfg, name, total):
    """Runs far longer than the pre-tokenizer's 64-byte halo, spread over an
    input of fewer than 1024 tiles (8-wave workgroups) and of more (4-wave
    workgroups): the run carries then come from blocks in global memory."""
    t, o, tokb = cfg[name]
    filler = textgen.mix_text(41, 300_000)
    runs = ["7" * 30_000, " " * 20_000, "\r\n" * 9_000, "x" + "\n" * 12_000 + "  y", "!" + " " * 9_000 + "\r\nz",
            "12" * 7_000, "\t " * 5_000 + "w"]
    parts, size, k = [], 0, 0
    while size < total:
        a = (k * 37_813) % 250_000
        piece = filler[a:a + 30_000 + 1_111 * (k % 5)] + runs[k % len(runs)]
        parts.append(piece)
        size += len(piece)
        k += 1
    b = "".join(parts).encode()
    want = o.encode(b)
    _check(f"{name}[{len(b)}]", t.encode(b), want, b, tokb)
    _check(f"{name}[{len(b)}] dev", gpu_encode_dev(t, b), want, b, tokb)


@pytest.mark.parametrize("name", ["tiny", "gpt2", "llama3"])
def test_long_pieces(cfg, name):
    t, o, tokb = cfg[name]
    rng = random.Random(7)
    cases = []
    for L in [33, 63, 64, 65, 100, 128, 129, 511, 512, 513, 4095, 4096, 4097, 10_000]:
        cases += ["a" * L, " " * L + "x", "=" * L, "é" * L, "\n" * L + "x", "中" * L,
                  "".join(rng.choice("abcdefghij") for _ in range(L)),
                  "".join(rng.choice("aab") for _ in range(L)), "7" * L, "x" + "1" * L]
    cases.append(" " + "ab" * 20000)
    text = "|".join(cases)
    b = text.encode()
    _check(name, t.encode(b), o.encode(b), b, tokb)
    for s in cases[::7]:
        bb = s.encode()
        _check(name, t.encode(bb), o.encode(bb), bb, tokb)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_long_pieces_in_batches(cfg, name):
    """Pieces over 64 bytes (merged by the long-piece kernel and expanded from
    one marker by the assembly) at document starts and ends, several in one
    tile, across tiles, on both sides of the 4,096-symbol LDS capacity: IDs and
    output offsets equal the oracle's per document."""
    t, o, tokb = cfg[name]
    rng = random.Random(99)
    cjk = lambda k: "".join(chr(rng.randint(0x4E00, 0x9FFF)) for _ in range(k))  # noqa: E731
    docs = ["a" * 65, " " * 200 + "x", cjk(40) + ". " + cjk(30), "x", "", "=" * 70 + " " + "-" * 66 + "\n",
            cjk(1365), cjk(1366) + "!", "ab" * 2100, "q " + "7" * 300, " " * 64 + "y", "é" * 33 + "z" * 64]
    docs += [cjk(rng.randint(20, 90)) + rng.choice([", ", ".\n", " ok "]) for _ in range(40)]
    data, off = textgen.pack_docs(docs)
    ids, out_off = t.encode_batch(data, off)
    want = [o.encode(d.encode()) for d in docs]
    want_ids, want_off = oracle_par.concat(want)
    assert np.array_equal(out_off, want_off), "output offsets differ"
    _check(name, ids, want_ids, data, tokb)


def test_empty_and_tiny_inputs(cfg):
    t, o, _ = cfg["gpt2"]
    assert len(t.encode(b"")) == 0
    for s in ["a", " ", "\n", "'", "'s", "é", "😀", "12", "a b", "  "]:
        assert np.array_equal(t.encode(s.encode()), o.encode(s.encode())), s


INVALID = [b"\xff", b"a\x80b", b"\xc3", b"ab\xc3", b"\xe0\x80\x80", b"\xed\xa0\x80", b"\xf4\x90\x80\x80",
           b"\xc0\xaf", b"\xc1\xbf", b"\xf5\x80\x80\x80", b"\xe2\x82", b"\xe2\x28\xa1", b"\xf0\x9f\x98",
           b"\x80", b"\xbf\xbf"]


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_invalid_utf8_rejected(cfg, name):
    t, o, _ = cfg[name]
    good = textgen.mix_text(8, 20_000).encode()
    for bad in INVALID:
        for b in (bad, good[:5000] + bad + good[5000:], good + bad):
            with pytest.raises(UnicodeDecodeError):
                o.encode(b)
            with pytest.raises(tk.TokError) as e:
                t.encode(b)
            assert e.value.code == tk.TOK_E_UTF8, (bad, len(b))


def test_capacity_overflow(cfg):
    t, o, _ = cfg["gpt2"]
    b = textgen.mix_text(9, 5000).encode()
    want = o.encode(b)
    d = dev_bytes(b)
    ids = torch.full((10,), -1, dtype=torch.int32, device="cuda")
    n = ctypes.c_size_t(0)
    rc = tk.lib().tok_encode_dev(t._h, d.data_ptr(), len(b), ids.data_ptr(), 10, ctypes.byref(n),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == tk.TOK_E_CAPACITY and n.value == len(want)
    assert np.array_equal(ids.cpu().numpy(), want[:10])
    host = np.full(5, -1, dtype=np.int32)
    rc = tk.lib().tok_encode(t._h, b, len(b), host.ctypes.data, 5, ctypes.byref(n))
    assert rc == tk.TOK_E_CAPACITY and n.value == len(want)
    assert (host == -1).all()


def batch_docs():
    docs = ["", "abc 123", "12", "345", "it'", "s fine", "tail   ", "\n  x", "", "中文", "😀😀", "",
            "x" + "9" * 5000, "  \n", "\n\n", "'S", "'s", " ", "a" * 300]
    docs += [textgen.mix_text(400 + i, 9000 + 1371 * i) for i in range(6)]
    docs += [""]
    return docs


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_batch_parity(cfg, name):
    t, o, tokb = cfg[name]
    data, off = textgen.pack_docs(batch_docs())
    want_ids, want_off = o.encode_batch(data, off)
    ids, out_off = t.encode_batch(data, off)
    assert np.array_equal(out_off, want_off)
    _check(name, ids, want_ids, data, tokb)
    # split level with document boundaries
    want_p = []
    for i in range(len(off) - 1):
        s, e = int(off[i]), int(off[i + 1])
        want_p += [s + p for p in o.pieces(data[s:e])]
    assert gpu_pieces(t, data, off) == want_p
    # device-resident batch
    d = dev_bytes(data)
    d_off = torch.tensor(off.astype(np.int64), device="cuda").view(torch.uint64)
    d_ids = torch.empty(len(data), dtype=torch.int32, device="cuda")
    d_out = torch.empty(len(off), dtype=torch.int64, device="cuda").view(torch.uint64)
    n = t.encode_batch_dev(d, d_off, d_ids, d_out)
    torch.cuda.synchronize()
    assert n == len(want_ids)
    assert np.array_equal(d_ids[:n].cpu().numpy(), want_ids)
    assert np.array_equal(d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)


def test_batch_rejects_bad_offsets(cfg):
    t, _, _ = cfg["gpt2"]
    data = b"hello world"
    for off in ([0, 5, 3, 11], [1, 11], [0, 5, 12]):
        arr = np.asarray(off, dtype=np.uint64)
        if off[-1] != len(data):
            # the host entry takes the length from the last offset; the device
            # entry checks it against the text it is given
            d = dev_bytes(data)
            d_off = torch.tensor(arr.astype(np.int64), device="cuda").view(torch.uint64)
            d_ids = torch.empty(32, dtype=torch.int32, device="cuda")
            d_out = torch.empty(len(off), dtype=torch.int64, device="cuda").view(torch.uint64)
            with pytest.raises(tk.TokError) as e:
                t.encode_batch_dev(d, d_off, d_ids, d_out)
            assert e.value.code == tk.TOK_E_ARG
        else:
            with pytest.raises(tk.TokError) as e:
                t.encode_batch(data, arr)
            assert e.value.code == tk.TOK_E_ARG
    with pytest.raises(tk.TokError):
        t.encode_batch(data, np.asarray([1, 11], dtype=np.uint64))


def test_batch_workload(cfg):
    """64 documents of 500,000 characters in one call (the batch workload):
    every document's IDs and output offsets equal the oracle's encode of that
    document, element by element."""
    t, o, tokb = cfg["llama3"]
    texts = textgen.batch_texts(40_000, 64, 500_000)
    data, off = textgen.pack_docs(texts)
    ids, out_off = t.encode_batch(data, off)
    docs = [data[int(off[i]):int(off[i + 1])] for i in range(64)]
    want_ids, want_off = oracle_par.concat(oracle_par.map_docs(o.encode, docs))
    assert np.array_equal(out_off, want_off), "output offsets differ"
    for i in range(64):
        a, z = int(out_off[i]), int(out_off[i + 1])
        _check(f"doc {i}", ids[a:z], want_ids[a:z], docs[i], tokb)
    assert np.array_equal(ids, want_ids)


def test_repair_seams(cfg):
    """Seam shapes that append repair meets (a word cut mid-run, newline plus
    spaces on both sides of the seam, a multibyte character's bytes at the
    seam): the encode of the concatenation equals the oracle."""
    t, o, tokb = cfg["gpt2"]
    for seed in range(6):
        old, suf = textgen.repair_case(100 + seed, 200 + seed, old_chars=20_000)
        b = (old + suf).encode()
        _check(f"seam {seed}", t.encode(b), o.encode(b), b, tokb)
    for s in ["watch the staging pipe" + "line closely.", "x\n  " + "\n   y", "命" * 3 + "令"]:
        b = s.encode()
        _check(s, t.encode(b), o.encode(b), b, tokb)


@pytest.mark.parametrize("poison", [None, 0xFF, 0x00, 0x5A])
def test_stale_state_across_sizes(cfg, poison):
    """Calls of different sizes on one context, with every per-call device
    buffer filled with a poison byte before each call (GraphTok, section 6.2:
    stale state across replays): the results never depend on what an earlier
    call or the poison left in the scratch."""
    t, o, tokb = cfg["llama3"]
    small = "x12345 it's\n\n  fine".encode()
    big = textgen.mix_text(12, 3_000_000).encode()
    want_small, want_big = o.encode(small), o.encode(big)
    docs = [big[:5000], b"", small, big[5000:90_000]]
    data, off = b"".join(docs), np.cumsum([0] + [len(d) for d in docs]).astype(np.uint64)
    want_batch = np.concatenate([o.encode(d) for d in docs])
    for b, w in ((small, want_small), (big, want_big), (small, want_small), (big[:777], o.encode(big[:777])),
                 (big, want_big)):
        if poison is not None:
            t.fill_scratch(poison)
        _check("stale", t.encode(b), w, b, tokb)
        if poison is not None:
            t.fill_scratch(poison)
        _check("stale-dev", gpu_encode_dev(t, b), w, b, tokb)
        if poison is not None:
            t.fill_scratch(poison)
        got, got_off = t.encode_batch(data, off)
        _check("stale-batch", got, want_batch, data, tokb)


def test_deterministic(cfg):
    t, _, _ = cfg["gpt2"]
    b = textgen.mix_text(13, 200_000).encode()
    a = t.encode(b)
    for _ in range(3):
        assert np.array_equal(t.encode(b), a)


def test_stage_timing_mask(cfg):
    """tok_set_profiling takes a stage mask: only the chosen stages get durations."""
    t, o, tokb = cfg["gpt2"]
    b = textgen.mix_text(14, 50_000).encode()
    d = dev_bytes(b)
    ids = torch.empty(len(b), dtype=torch.int32, device="cuda")
    t.set_profiling(True)
    t.encode_dev(d, ids)
    ms = t.stage_ms()
    assert len(ms) == len(tk.STAGES) and all(x > 0 for x in ms)
    t.set_profiling(1 << tk.STAGES.index("pieces"))
    n = t.encode_dev(d, ids)
    ms = t.stage_ms()
    assert ms[tk.STAGES.index("pieces")] > 0
    assert all(x == 0 for i, x in enumerate(ms) if i != tk.STAGES.index("pieces"))
    t.set_profiling(False)
    _check("timed", ids[:n].cpu().numpy(), o.encode(b), b, tokb)


def test_all_empty_batch(cfg):
    """Every document empty: no tile runs; offsets are all zero (host and device
    entry), and a nonzero offset in an empty text is rejected on the device."""
    t, _, _ = cfg["llama3"]
    off = np.zeros(6, dtype=np.uint64)
    ids, out_off = t.encode_batch(b"", off)
    assert len(ids) == 0 and (out_off == 0).all()
    d = torch.empty(0, dtype=torch.uint8, device="cuda")
    d_ids = torch.empty(1, dtype=torch.int32, device="cuda")
    for good, arr in ((True, off), (False, np.array([0, 0, 1, 0], dtype=np.uint64))):
        d_off = torch.tensor(arr.astype(np.int64), device="cuda").view(torch.uint64)
        d_out = torch.full((len(arr),), 7, dtype=torch.int64, device="cuda").view(torch.uint64)
        if good:
            assert t.encode_batch_dev(d, d_off, d_ids, d_out) == 0
            assert (d_out.view(torch.int64).cpu().numpy() == 0).all()
        else:
            with pytest.raises(tk.TokError) as e:
                t.encode_batch_dev(d, d_off, d_ids, d_out)
            assert e.value.code == tk.TOK_E_ARG


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_many_tiny_documents(cfg, name):
    """Thousands of 0..5-byte documents: many document starts per tile and per
    16-byte chunk, and more documents than threads in a workgroup."""
    t, o, tokb = cfg[name]
    rng = random.Random(77)
    alpha = ["a", "b", " ", "1", "'", "s", "\n", "é", ".", "😀"]
    docs = ["".join(rng.choice(alpha) for _ in range(rng.randint(0, 3))) for _ in range(6000)]
    data, off = textgen.pack_docs(docs)
    want_ids, want_off = o.encode_batch(data, off)
    ids, out_off = t.encode_batch(data, off)
    assert np.array_equal(out_off, want_off)
    _check(name, ids, want_ids, data, tokb)


FUZZ_ALPHA = (list("abcdefghijklmnopqrstuvwxyzSTRVMLD") + list("0123456789") + [" ", "  ", "\t", "\n", "\r",
              "\r\n", " ", "\u0085", " ", "　"] + list(".,;:!?'\"()[]{}<>=+-*/\\|&^%$#@~`_") +
              ["é", "ß", "ſ", "Ω", "中", "文", "ひ", "한", "́", "²", "½", "Ⅳ", "😀", "🧪", "\U0001F1FA"])


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_random_texts(cfg, name):
    """Seeded random texts over a rich alphabet (letters, contraction letters in
    both cases, digits, every whitespace kind, punctuation, accents, CJK,
    combining marks, other number forms, emoji), with runs, as one batch and as
    single requests."""
    t, o, tokb = cfg[name]
    rng = random.Random(1234 if name == "gpt2" else 4321)
    docs = []
    for _ in range(400):
        n = rng.choice([0, 1, 2, 5, 17, 64, 300, 1500, 5000])
        parts = []
        while len(parts) < n:
            tok = rng.choice(FUZZ_ALPHA)
            parts.append(tok * rng.choice([1, 1, 1, 2, 3, 8, 70]))
        docs.append("".join(parts))
    data, off = textgen.pack_docs(docs)
    want_ids, want_off = o.encode_batch(data, off)
    ids, out_off = t.encode_batch(data, off)
    assert np.array_equal(out_off, want_off)
    _check(name, ids, want_ids, data, tokb)
    for s in docs[:60]:
        b = s.encode()
        _check(name, t.encode(b), o.encode(b), b, tokb)
    whole = "".join(docs).encode()
    _check(name, t.encode(whole), o.encode(whole), whole, tokb)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_unaligned_device_text(cfg, name):
    """Text that starts 1, 2 or 3 bytes into a device buffer: the kernels
    fall back from word loads to byte loads, with the same result; the batch
    call and the literal pass too."""
    t, o, _ = cfg[name]
    b = textgen.mix_text(66, 50_000).encode()
    want = o.encode(b)
    v = t.info()["vocab_size"]
    lits = [(b"<|x|>", v), (b"=>", v + 1)]
    data, off = textgen.pack_docs([b[:20_000].decode(errors="ignore"), "", b[20_000:].decode(errors="ignore")])
    want_b, want_off = o.encode_batch(data, off)
    for shift in (1, 2, 3):
        d = torch.frombuffer(bytearray(b"\0" * shift + b), dtype=torch.uint8).cuda()[shift:]
        assert d.data_ptr() % 4 == shift
        ids = torch.empty(len(b), dtype=torch.int32, device="cuda")
        n = t.encode_dev(d, ids)
        torch.cuda.synchronize()
        _check(f"{name}+{shift}", ids[:n].cpu().numpy(), want, b, None)
        db = torch.frombuffer(bytearray(b"\0" * shift + data), dtype=torch.uint8).cuda()[shift:]
        d_off = torch.tensor(off.astype(np.int64), device="cuda").view(torch.uint64)
        d_out = torch.empty(len(off), dtype=torch.int64, device="cuda").view(torch.uint64)
        d_ids = torch.empty(len(data), dtype=torch.int32, device="cuda")
        n = t.encode_batch_dev(db, d_off, d_ids, d_out)
        torch.cuda.synchronize()
        _check(f"{name}+{shift} batch", d_ids[:n].cpu().numpy(), want_b, data, None)
        assert np.array_equal(d_out.view(torch.int64).cpu().numpy().astype(np.uint64), want_off)
        t.set_added_tokens(lits)
        try:
            n = t.encode_dev(d, ids)
            torch.cuda.synchronize()
            _check(f"{name}+{shift} literals", ids[:n].cpu().numpy(), o.encode_added(b, lits), b, None)
        finally:
            t.set_added_tokens([])


def test_too_long_rejected(cfg):
    """A length past TOK_MAX_BYTES is refused with TOK_E_TOOLONG by every entry
    point before any buffer is read or written (the buffers here are small;
    only the stated length is out of range)."""
    t, _, _ = cfg["gpt2"]
    big = tk.TOK_MAX_BYTES + 1
    s = torch.cuda.current_stream().cuda_stream
    d_text = torch.zeros(64, dtype=torch.uint8, device="cuda")
    d_ids = torch.full((64,), -1, dtype=torch.int32, device="cuda")
    d_spans = torch.zeros(64, dtype=torch.int32, device="cuda")
    d_flags = torch.zeros(64, dtype=torch.int16, device="cuda")
    d_doc = torch.tensor([0, big], dtype=torch.int64, device="cuda")
    d_out = torch.zeros(2, dtype=torch.int64, device="cuda")
    host_text = bytes(64)
    host_ids = np.full(64, -1, dtype=np.int32)
    host_spans = np.zeros(64, dtype=np.uint32)
    doc = np.array([0, big], dtype=np.uint64)
    out = np.zeros(2, dtype=np.uint64)
    n = ctypes.c_size_t(7)
    L = tk.lib()
    calls = {
        "tok_encode": lambda: L.tok_encode(t._h, host_text, big, host_ids.ctypes.data, 64, ctypes.byref(n)),
        "tok_encode_dev": lambda: L.tok_encode_dev(t._h, d_text.data_ptr(), big, d_ids.data_ptr(), 64,
                                                   ctypes.byref(n), s),
        "tok_encode_batch": lambda: L.tok_encode_batch(t._h, host_text, doc.ctypes.data, 1, host_ids.ctypes.data,
                                                       64, out.ctypes.data),
        "tok_encode_batch_dev": lambda: L.tok_encode_batch_dev(t._h, d_text.data_ptr(), big, d_doc.data_ptr(), 1,
                                                               d_ids.data_ptr(), 64, d_out.data_ptr(),
                                                               ctypes.byref(n), s),
        "tok_encode_spans": lambda: L.tok_encode_spans(t._h, host_text, big, host_ids.ctypes.data,
                                                       host_spans.ctypes.data, 64, ctypes.byref(n)),
        "tok_encode_spans_dev": lambda: L.tok_encode_spans_dev(t._h, d_text.data_ptr(), big, None, 0,
                                                               d_ids.data_ptr(), d_spans.data_ptr(), 64, None,
                                                               ctypes.byref(n), s),
        "tok_pretokenize_dev": lambda: L.tok_pretokenize_dev(t._h, d_text.data_ptr(), big, None, 0,
                                                             d_flags.data_ptr(), s),
        "tok_repair": lambda: L.tok_repair(t._h, host_ids.ctypes.data, 0, 64, host_text, 0, big, ctypes.byref(n),
                                           None),
        "tok_repair_dev": lambda: L.tok_repair_dev(t._h, d_ids.data_ptr(), 0, 64, host_text, 0, big,
                                                   ctypes.byref(n), None),
    }
    for name, call in calls.items():
        n.value = 7
        assert call() == tk.TOK_E_TOOLONG, name
        if name not in ("tok_encode_batch", "tok_pretokenize_dev"):  # these have no count argument
            assert n.value == 0, name
    torch.cuda.synchronize()
    assert (host_ids == -1).all() and (d_ids.cpu().numpy() == -1).all()
