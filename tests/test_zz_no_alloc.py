"""tok_encode_dev_noalloc: the entry point that allocates nothing, for callers
that cannot allocate device memory during a call.  Its buffers come from one
fixed device array; its results must equal tok_encode_dev's (which grows its
own scratch) and the oracle's, element by element, on consecutive calls
(the second smaller than the first, so stale contents of the shared array
would show), up to the stated maximum input, and it must refuse a longer
input and a context with added-token literals before touching any buffer."""
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
    for name in ("gpt2", "llama3", "o200k"):
        merges_name, pattern = libs.CONFIGS[name]
        m = vocab.merges(merges_name)
        out[name] = (tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern))
    return out


def run_both(t, b: bytes):
    d = torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()
    a = torch.full((len(b) + 8,), -3, dtype=torch.int32, device="cuda")
    z = torch.full((len(b) + 8,), -5, dtype=torch.int32, device="cuda")
    n1 = t.encode_dev(d, a)
    n2 = t.encode_dev_noalloc(d, z)
    torch.cuda.synchronize()
    return a[:n1].cpu().numpy(), z[:n2].cpu().numpy(), z[n2:].cpu().numpy()


@pytest.mark.parametrize("name", ["gpt2", "llama3", "o200k"])
def test_noalloc_matches_encode_dev(cfg, name):
    t, o = cfg[name]
    big = textgen.mix_text(61, 1_100_000).encode()[: tk.TOK_NOALLOC_MAX_BYTES]
    while big and (big[-1] & 0xC0) == 0x80:  # whole code points only
        big = big[:-1]
    if big and big[-1] >= 0xC0:
        big = big[:-1]
    cjk = textgen.cjk_text(62, 40_000).encode()
    small = textgen.mix_text(63, 3_000).encode()
    # stretches without a cut across tiles: under the case-splitting family the
    # tiles hand their cursors over through words in the shared array
    stretch = ("q " + "7" * 20_000 + " " * 5_000 + "x'd" * 3_000 + " z").encode()
    for b in (big, small, cjk, b"x", stretch, small[:1000]):
        ref, got, tail = run_both(t, b)
        assert np.array_equal(got, ref), len(b)
        assert np.all(tail == -5), "nothing written past the count"
        if len(b) <= 50_000:
            assert np.array_equal(got, o.encode(b)), len(b)


def test_noalloc_limits(cfg):
    t, _ = cfg["gpt2"]
    n = tk.TOK_NOALLOC_MAX_BYTES + 1
    d = torch.full((n,), ord("a"), dtype=torch.uint8, device="cuda")
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    with pytest.raises(tk.TokError) as e:
        t.encode_dev_noalloc(d, ids)
    assert e.value.code == tk.TOK_E_TOOLONG
    v = t.info()["vocab_size"]
    t.set_added_tokens([(b"<|x|>", v)])
    try:
        with pytest.raises(tk.TokError) as e:
            t.encode_dev_noalloc(d[:100], ids)
        assert e.value.code == tk.TOK_E_ARG
    finally:
        t.set_added_tokens([])
    # malformed UTF-8 and a small output buffer report as tok_encode_dev does
    bad = torch.frombuffer(bytearray(b"ab\xffcd"), dtype=torch.uint8).cuda()
    with pytest.raises(tk.TokError) as e:
        t.encode_dev_noalloc(bad, ids)
    assert e.value.code == tk.TOK_E_UTF8
    text = torch.frombuffer(bytearray(textgen.mix_text(64, 5000).encode()), dtype=torch.uint8).cuda()
    with pytest.raises(tk.TokError) as e:
        t.encode_dev_noalloc(text, ids[:10])
    assert e.value.code == tk.TOK_E_CAPACITY
