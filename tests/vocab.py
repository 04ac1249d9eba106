"""Test helpers: the committed merge lists and their token byte strings."""
import hashlib
import json
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
VOCAB_DIR = os.path.join(ROOT, "synth", "vocab")
MANIFEST = json.load(open(os.path.join(VOCAB_DIR, "manifest.json")))


def merges(name: str) -> np.ndarray:
    path = os.path.join(VOCAB_DIR, MANIFEST[name]["file"])
    raw = open(path, "rb").read()
    assert hashlib.sha256(raw).hexdigest() == MANIFEST[name]["sha256"], f"{name} artifact changed"
    return np.frombuffer(raw, dtype="<u4").reshape(-1, 2).copy()


def token_bytes(m: np.ndarray) -> list:
    """bytes of every ID: byte b -> bytes([b]); merge r -> tok[left] + tok[right]."""
    tok = [bytes([b]) for b in range(256)]
    for a, b in m.tolist():
        tok.append(tok[a] + tok[b])
    return tok


def detok(ids, tok) -> bytes:
    return b"".join(tok[i] for i in ids)
