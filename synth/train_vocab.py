"""Train the seeded merge lists (the frozen tokenizer configurations).

    python -m synth.train_vocab [--only tiny_1k|gpt2_50k|llama3_128k|o200k_64k]

For each vocabulary: generate the seeded training corpus (synth.textgen),
split it into pieces with the third-party ``regex`` module running the
family's published pattern, count piece frequencies, and run the C++ greedy
trainer (synth/bpe_train.cpp).  Writes ``synth/vocab/<name>.merges`` (uint32
left, right per merge, in rank order; merge r creates ID 256 + r) and records
its SHA-256 in ``synth/vocab/manifest.json``.

The training split uses the ``regex`` module, not the oracle and not the GPU
path: a merge list is an input to both, and any list is a valid configuration.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import struct
import subprocess
import sys
import time
from multiprocessing import Pool

HERE = os.path.dirname(os.path.abspath(__file__))
VOCAB_DIR = os.path.join(HERE, "vocab")
CORPUS_DIR = os.path.join(HERE, "_corpus")

# The two split patterns, written from the family descriptions (GPT-2 style:
# contractions, optional space + letters / digits / other, whitespace
# lookahead; Llama-3 style: case-insensitive contractions, optional
# non-letter/non-digit prefix, digit groups of 1-3, newline-aware whitespace).
PATTERNS = {
    "gpt2": r"""'s|'t|'re|'ve|'m|'ll|'d| ?\p{L}+| ?\p{N}+| ?[^\s\p{L}\p{N}]+|\s+(?!\S)|\s+""",
    "llama3": r"""(?i:'s|'t|'re|'ve|'m|'ll|'d)|[^\r\n\p{L}\p{N}]?\p{L}+|\p{N}{1,3}| ?[^\s\p{L}\p{N}]+[\r\n]*|\s*[\r\n]+|\s+(?!\S)|\s+""",
    # case-splitting style, composed from TokTier's description of the o200k
    # lineage (section 4, "Removing the sequential regex scan"): the Llama-3
    # style with letter runs split at case boundaries (an optional run of
    # upper-case or caseless letters or marks, then lower-case or caseless
    # letters or marks), marks joining letters, and the contractions as an
    # optional suffix of a letter piece
    "o200k": (r"""[^\r\n\p{L}\p{N}]?[\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}]*[\p{Ll}\p{Lm}\p{Lo}\p{M}]+"""
              r"""(?i:'s|'t|'re|'ve|'m|'ll|'d)?"""
              r"""|[^\r\n\p{L}\p{N}]?[\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}]+[\p{Ll}\p{Lm}\p{Lo}\p{M}]*"""
              r"""(?i:'s|'t|'re|'ve|'m|'ll|'d)?"""
              r"""|\p{N}{1,3}| ?[^\s\p{L}\p{N}]+[\r\n]*|\s*[\r\n]+|\s+(?!\S)|\s+"""),
}

# name -> (generator, corpus seeds, chars per doc, pattern, merges)
VOCABS = {
    "tiny_1k": ("tiny", [101], 200_000, "gpt2", 1_000),
    "gpt2_50k": ("mix", list(range(20_000, 20_020)), 1_000_000, "gpt2", 50_000),
    "llama3_128k": ("mix", list(range(50_000, 50_050)), 1_000_000, "llama3", 127_744),
    "o200k_64k": ("mix", list(range(80_000, 80_020)), 1_000_000, "o200k", 64_000),
}


def _count_doc(args):
    gen, seed, n_chars, pattern = args
    import regex

    sys.path.insert(0, os.path.dirname(HERE))
    from synth import textgen

    text = textgen.tiny_text(seed, n_chars) if gen == "tiny" else textgen.mix_text(seed, n_chars)
    c = collections.Counter(regex.findall(PATTERNS[pattern], text))
    return {k.encode("utf-8"): v for k, v in c.items()}


def build_trainer() -> str:
    os.makedirs(CORPUS_DIR, exist_ok=True)
    exe = os.path.join(CORPUS_DIR, "bpe_train")
    src = os.path.join(HERE, "bpe_train.cpp")
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(src):
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-o", exe, src])
    return exe


def train(name: str, workers: int = 8) -> dict:
    gen, seeds, n_chars, pattern, n_merges = VOCABS[name]
    t0 = time.time()
    total = collections.Counter()
    with Pool(min(workers, len(seeds))) as pool:
        for c in pool.imap(_count_doc, [(gen, s, n_chars, pattern) for s in seeds]):
            total.update(c)
    t1 = time.time()
    os.makedirs(CORPUS_DIR, exist_ok=True)
    words_path = os.path.join(CORPUS_DIR, f"{name}.words")
    with open(words_path, "wb") as f:
        items = sorted(total.items())
        f.write(struct.pack("<Q", len(items)))
        for k, v in items:
            f.write(struct.pack("<QI", v, len(k)))
            f.write(k)
    exe = build_trainer()
    out = os.path.join(VOCAB_DIR, f"{name}.merges")
    subprocess.check_call([exe, words_path, str(n_merges), out])
    t2 = time.time()
    with open(out, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    info = {
        "file": f"{name}.merges",
        "sha256": digest,
        "n_merges": n_merges,
        "pattern": pattern,
        "generator": gen,
        "corpus_seeds": [seeds[0], seeds[-1]],
        "corpus_chars": n_chars * len(seeds),
        "distinct_pieces": len(total),
        "tie_break": "max count, then smallest (left_id, right_id); skip pairs whose bytes are already a token",
    }
    print(f"{name}: {len(total)} distinct pieces, split {t1 - t0:.1f}s, train {t2 - t1:.1f}s, sha256 {digest}")
    return info


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", default=None)
    args = ap.parse_args()
    os.makedirs(VOCAB_DIR, exist_ok=True)
    man_path = os.path.join(VOCAB_DIR, "manifest.json")
    manifest = json.load(open(man_path)) if os.path.exists(man_path) else {}
    for name in VOCABS:
        if args.only and name != args.only:
            continue
        manifest[name] = train(name)
        with open(man_path, "w") as f:
            json.dump(manifest, f, indent=2, sort_keys=True)


if __name__ == "__main__":
    main()
