"""GPU parity on CJK-dense text, where every ideograph run is one letter
piece of up to 6,000 bytes (TokTier, Table 9 reports CJK corpora apart;
GraphTok, section 6.2: long pre-tokens).  The pipeline cuts them into units
of BPE where no token spans the byte pair; the units over 64 bytes take the
long-piece merge path.

The oracle's textbook BPE is quadratic in a piece's length, so whole texts
are compared element by element at sizes it finishes in seconds (runs still
span several tiles).  At the workload's full size (1,000,000 characters) the
pieces are taken from the oracle's own pre-tokenizer, and sampled pieces
(the longest ones and a seeded random draw) are compared one by one: the
GPU's tokens whose spans fall in a piece must equal the oracle's BPE of the
piece's bytes.  Every token of the full output must also spell its bytes.
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
    for name in ("gpt2", "llama3"):
        merges_name, pattern = libs.CONFIGS[name]
        m = vocab.merges(merges_name)
        out[name] = (tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern), vocab.token_bytes(m))
    return out


def dev_spans(t, b: bytes):
    d = torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()
    ids = torch.full((len(b),), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((len(b),), -7, dtype=torch.int32, device="cuda")
    n = t.encode_spans_dev(d, ids, sp)
    torch.cuda.synchronize()
    return ids[:n].cpu().numpy(), sp[:n].cpu().numpy().view(np.uint32).astype(np.int64)


def same(what, got, want):
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape or not np.array_equal(got, want):
        n = min(len(got), len(want))
        i = next((k for k in range(n) if got[k] != want[k]), n)
        pytest.fail(f"{what}: {len(got)} vs {len(want)} IDs, first difference at {i}: "
                    f"gpu {got[i:i + 6].tolist()} oracle {want[i:i + 6].tolist()}")


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
@pytest.mark.parametrize("seed,n_chars", [(11, 3_000), (12, 12_000)])
def test_cjk_small_exact(cfg, name, seed, n_chars):
    t, o, _ = cfg[name]
    b = textgen.cjk_text(seed, n_chars).encode()
    same(f"cjk {seed}", t.encode(b), o.encode(b))
    ids, sp = dev_spans(t, b)
    want_ids, want_sp = o.encode_spans(b)
    same(f"cjk {seed} device ids", ids, want_ids)
    same(f"cjk {seed} spans", sp, want_sp.astype(np.int64))


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_cjk_workload_sampled_pieces(cfg, name):
    """The 1,000,000-character CJK-dense workload: sampled pieces equal the
    oracle's BPE of their bytes; all tokens tile the input."""
    t, o, tokb = cfg[name]
    b = textgen.cjk_text(5, 1_000_000).encode()
    ids, sp = dev_spans(t, b)
    lens = np.asarray([len(x) for x in tokb], dtype=np.int64)[ids]
    assert sp[0] == 0 and np.array_equal(sp[1:], sp[:-1] + lens[:-1]) and sp[-1] + lens[-1] == len(b)
    starts = np.asarray(o.pieces(b) + [len(b)], dtype=np.int64)
    plen = np.diff(starts)
    order = np.argsort(-plen, kind="stable")
    rng = random.Random(77)
    pick = sorted(set(order[:8].tolist()) | set(rng.sample(range(len(plen)), 24)))
    wants = oracle_par.map_docs(lambda i: o.bpe(b[starts[i]:starts[i + 1]]), pick)
    for i, want in zip(pick, wants):
        a, z = np.searchsorted(sp, [starts[i], starts[i + 1]])
        same(f"piece {i} ({plen[i]} bytes at {starts[i]})", ids[a:z], want)


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_cjk_split_is_the_pattern_alone(cfg, name):
    """The pipeline cuts long ideograph runs into units of BPE where no token
    spans the byte pair; the pre-tokenization entry point still returns the
    pattern's pieces alone."""
    t, o, _ = cfg[name]
    b = textgen.cjk_text(13, 200_000).encode()
    d = torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()
    flags = torch.zeros((len(b) + 15) // 16 + 8, dtype=torch.int16, device="cuda")
    t.pretokenize_dev(d, flags)
    torch.cuda.synchronize()
    same("pieces", tk.flags_to_starts(flags.cpu().numpy().view(np.uint16), len(b)), o.pieces(b))
