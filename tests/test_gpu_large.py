"""Large inputs: a request of just over 1 GiB through the device path, checked
against the oracle exactly.

The text is one 1,000,000-character block repeated.  Each block starts with a
digit and ends with a letter, so every seam is a letter -> digit class change,
a synchronizing transition for both pattern families (pieces from the seam on
do not depend on the text before it, and pieces before it do not depend on
the text after it).  The encode of the whole text is therefore the oracle's
encode of one block, repeated, which the oracle computes in a fraction of a
second.  This covers byte offsets above 2^30, more than a million 1 KiB
tiles, and both levels of tile-count groups in the output assembly.
"""
import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("name", ["gpt2", "llama3"])
def test_gigabyte_request(name):
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    merges_name, pattern = libs.CONFIGS[name]
    m = vocab.merges(merges_name)
    t, o = tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern)
    block = ("1" + textgen.mix_text(77, 999_998) + "x").encode()
    copies = (1 << 30) // len(block) + 2
    want_block = o.encode(block)
    d_block = torch.frombuffer(bytearray(block), dtype=torch.uint8).cuda()
    d_text = d_block.repeat(copies)
    n = d_text.numel()
    assert n > (1 << 30)
    ids = torch.empty(n // 2, dtype=torch.int32, device="cuda")
    count = t.encode_dev(d_text, ids)
    torch.cuda.synchronize()
    assert count == len(want_block) * copies, (count, len(want_block), copies)
    got = ids[:count].view(copies, len(want_block))
    want = torch.from_numpy(want_block).cuda()
    bad = (got != want.unsqueeze(0)).any(dim=1).nonzero().flatten().tolist()
    assert not bad, f"{name}: copies {bad[:5]} differ from the block's encode"
    del got, ids, d_text
    t.close()
    torch.cuda.empty_cache()
