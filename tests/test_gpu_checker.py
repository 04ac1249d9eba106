"""Checker mutation test: the parity check catches every planted fault.

TokTier (section 5.2, "Exactness") plants five kinds of fault in correct
outputs to show its checker catches them: an ID substituted, deleted or
duplicated, two adjacent IDs swapped, and a tail resplit into different
tokens of the same bytes and count.  Here the faults are planted in the
GPU's own output for a request (after it has been shown equal to the
oracle's), and the element-by-element comparison the parity tests use must
flag every mutated copy.  A resplit keeps the bytes, so the weaker check
"the tokens' bytes concatenate to the input" passes it: the control shows
why the parity tests compare IDs.
"""
import random

import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
import oracle
from synth import textgen
from tests import libs, vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def ids_equal(got, want) -> bool:
    """The parity tests' check: same length, same ID at every position."""
    got, want = np.asarray(got), np.asarray(want)
    return got.shape == want.shape and bool(np.array_equal(got, want))


def bytes_roundtrip(ids, tokb, text: bytes) -> bool:
    return b"".join(tokb[i] for i in ids) == text


def resplits(ids, tokb, by_bytes):
    """Positions i where tokens i, i + 1 re-split into two other vocabulary
    tokens of the same bytes, with the replacement pair."""
    out = []
    for i in range(len(ids) - 1):
        joint = tokb[ids[i]] + tokb[ids[i + 1]]
        for cut in range(1, len(joint)):
            if cut == len(tokb[ids[i]]):
                continue
            a, b = by_bytes.get(joint[:cut]), by_bytes.get(joint[cut:])
            if a is not None and b is not None:
                out.append((i, a, b))
                break
    return out


def test_every_planted_fault_is_flagged():
    libs.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    merges_name, pattern = libs.CONFIGS["gpt2"]
    m = vocab.merges(merges_name)
    t, o = tk.Tokenizer(m, pattern), oracle.Oracle(m, pattern)
    tokb = vocab.token_bytes(m)
    by_bytes = {b: i for i, b in enumerate(tokb)}
    text = textgen.mix_text(81, 60_000).encode()
    d = torch.frombuffer(bytearray(text), dtype=torch.uint8).cuda()
    buf = torch.empty(len(text) + 8, dtype=torch.int32, device="cuda")
    k = t.encode_dev(d, buf)
    gpu = buf[:k].cpu().numpy().tolist()
    want = o.encode(text).tolist()
    assert ids_equal(gpu, want), "the output to mutate must be correct"

    rng = random.Random(82)
    cand = resplits(gpu, tokb, by_bytes)
    assert len(cand) > 50
    counts = dict.fromkeys(["substitution", "deletion", "duplication", "adjacent swap", "tail resplit"], 0)
    for _ in range(200):
        i = rng.randrange(len(gpu))
        sub = list(gpu)
        sub[i] = (sub[i] + rng.randrange(1, len(tokb))) % len(tokb)
        dele = gpu[:i] + gpu[i + 1:]
        dup = gpu[:i + 1] + gpu[i:]
        j = next(j % (len(gpu) - 1) for j in range(i, i + len(gpu))
                 if gpu[j % (len(gpu) - 1)] != gpu[j % (len(gpu) - 1) + 1])  # two different IDs
        swap = list(gpu)
        swap[j], swap[j + 1] = swap[j + 1], swap[j]
        p, a, b = cand[rng.randrange(len(cand))]
        resplit = gpu[:p] + [a, b] + gpu[p + 2:]
        for kind, mutated in [("substitution", sub), ("deletion", dele), ("duplication", dup),
                              ("adjacent swap", swap), ("tail resplit", resplit)]:
            assert not ids_equal(mutated, want), (kind, i)
            counts[kind] += 1
        # the control: a resplit keeps the bytes, so a round-trip check passes it
        assert bytes_roundtrip(resplit, tokb, text) and len(resplit) == len(gpu)
    assert all(c == 200 for c in counts.values()), counts
