"""ctypes binding of the CPU oracle (oracle/oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  The oracle is plain,
single-threaded C++ that shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
PAT_GPT2, PAT_LLAMA3, PAT_O200K = 0, 1, 2
PATTERNS = {"gpt2": PAT_GPT2, "llama3": PAT_LLAMA3, "o200k": PAT_O200K}


class OracleError(RuntimeError):
    pass


def build() -> str:
    """Compile liboracle.so with g++ (always; callers decide when)."""
    src = os.path.join(HERE, "oracle.cpp")
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-o", tmp, src])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, u8p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
        L.orc_class.argtypes = [ctypes.c_uint32]
        L.orc_class.restype = ctypes.c_int
        L.orc_class_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp]
        L.orc_class_range.restype = None
        L.orc_subclass_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp]
        L.orc_subclass_range.restype = None
        L.orc_new.argtypes = [vp, sz, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        L.orc_new.restype = vp
        L.orc_free.argtypes = [vp]
        L.orc_free.restype = None
        for fn in (L.orc_pieces, L.orc_bpe, L.orc_encode):
            fn.argtypes = [vp, u8p, sz, vp, sz, ctypes.POINTER(sz)]
            fn.restype = ctypes.c_int
        L.orc_encode_batch.argtypes = [vp, u8p, vp, sz, vp, sz, vp]
        L.orc_encode_batch.restype = ctypes.c_int
        L.orc_encode_batch_spans.argtypes = [vp, u8p, vp, sz, vp, vp, sz, vp]
        L.orc_encode_batch_spans.restype = ctypes.c_int
        L.orc_encode_added.argtypes = [vp, u8p, vp, sz, vp, u8p, sz, vp, sz, ctypes.POINTER(sz)]
        L.orc_encode_added.restype = ctypes.c_int
        _lib = L
    return _lib


def char_class(cp: int) -> int:
    """0 = L, 1 = N, 2 = W, 3 = O."""
    return lib().orc_class(cp)


def class_range(lo: int, n: int) -> np.ndarray:
    """Classes of code points lo .. lo + n - 1 (uint8: 0 = L, 1 = N, 2 = W, 3 = O)."""
    out = np.zeros(n, dtype=np.uint8)
    lib().orc_class_range(lo, n, out.ctypes.data)
    return out


def subclass_range(lo: int, n: int) -> np.ndarray:
    """Subclasses of code points lo .. lo + n - 1 (uint8: 0 = U (Lu, Lt), 1 = D (Ll),
    2 = C (Lm, Lo), 3 = M (marks), 4 = N, 5 = W, 6 = O)."""
    out = np.zeros(n, dtype=np.uint8)
    lib().orc_subclass_range(lo, n, out.ctypes.data)
    return out


def load_merges(path: str) -> np.ndarray:
    m = np.fromfile(path, dtype="<u4")
    return m.reshape(-1, 2)


class Oracle:
    """Reference encoder for one (merges, pattern) configuration."""

    def __init__(self, merges, pattern):
        m = np.ascontiguousarray(np.asarray(merges, dtype=np.uint32).reshape(-1, 2))
        pat = PATTERNS[pattern] if isinstance(pattern, str) else int(pattern)
        err = ctypes.c_int(0)
        self._h = lib().orc_new(m.ctypes.data, m.shape[0], pat, ctypes.byref(err))
        if not self._h:
            raise OracleError(f"invalid merges or pattern (code {err.value})")
        self.n_merges = m.shape[0]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_free(h)
            self._h = None

    @staticmethod
    def _bytes(text) -> bytes:
        return text.encode("utf-8") if isinstance(text, str) else bytes(text)

    def pieces(self, text) -> list[int]:
        """Byte offsets where pieces start."""
        b = self._bytes(text)
        out = np.zeros(max(len(b), 1), dtype=np.uint64)
        n = ctypes.c_size_t(0)
        rc = lib().orc_pieces(self._h, b, len(b), out.ctypes.data, out.size, ctypes.byref(n))
        if rc:
            raise OracleError(f"pieces failed (code {rc})")
        return out[: n.value].tolist()

    def piece_strings(self, text) -> list[bytes]:
        b = self._bytes(text)
        st = self.pieces(b) + [len(b)]
        return [b[st[i]:st[i + 1]] for i in range(len(st) - 1)]

    def bpe(self, piece: bytes) -> list[int]:
        out = np.zeros(max(len(piece), 1), dtype=np.int32)
        n = ctypes.c_size_t(0)
        rc = lib().orc_bpe(self._h, piece, len(piece), out.ctypes.data, out.size, ctypes.byref(n))
        if rc:
            raise OracleError(f"bpe failed (code {rc})")
        return out[: n.value].tolist()

    def encode(self, text) -> np.ndarray:
        b = self._bytes(text)
        out = np.zeros(max(len(b), 1), dtype=np.int32)
        n = ctypes.c_size_t(0)
        rc = lib().orc_encode(self._h, b, len(b), out.ctypes.data, out.size, ctypes.byref(n))
        if rc == 1:
            raise UnicodeDecodeError("utf-8", b, 0, len(b), "invalid UTF-8 (oracle)")
        if rc:
            raise OracleError(f"encode failed (code {rc})")
        return out[: n.value].copy()

    def encode_batch(self, data: bytes, doc_off) -> tuple[np.ndarray, np.ndarray]:
        off = np.ascontiguousarray(np.asarray(doc_off, dtype=np.uint64))
        n_docs = off.size - 1
        out = np.zeros(max(len(data), 1), dtype=np.int32)
        out_off = np.zeros(n_docs + 1, dtype=np.uint64)
        rc = lib().orc_encode_batch(self._h, data, off.ctypes.data, n_docs, out.ctypes.data,
                                    out.size, out_off.ctypes.data)
        if rc == 1:
            raise UnicodeDecodeError("utf-8", data, 0, len(data), "invalid UTF-8 (oracle)")
        if rc:
            raise OracleError(f"encode_batch failed (code {rc})")
        return out[: int(out_off[-1])].copy(), out_off

    def encode_batch_spans(self, data: bytes, doc_off) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(ids, spans, out_off): spans[k] is the byte of data where token k starts, tracked
        through the merges themselves (a merged token starts where its left operand did)."""
        off = np.ascontiguousarray(np.asarray(doc_off, dtype=np.uint64))
        n_docs = off.size - 1
        out = np.zeros(max(len(data), 1), dtype=np.int32)
        spans = np.zeros(max(len(data), 1), dtype=np.uint64)
        out_off = np.zeros(n_docs + 1, dtype=np.uint64)
        rc = lib().orc_encode_batch_spans(self._h, data, off.ctypes.data, n_docs, out.ctypes.data,
                                          spans.ctypes.data, out.size, out_off.ctypes.data)
        if rc == 1:
            raise UnicodeDecodeError("utf-8", data, 0, len(data), "invalid UTF-8 (oracle)")
        if rc:
            raise OracleError(f"encode_batch_spans failed (code {rc})")
        t = int(out_off[-1])
        return out[:t].copy(), spans[:t].copy(), out_off

    def encode_spans(self, text) -> tuple[np.ndarray, np.ndarray]:
        """(ids, spans) of one text: spans[k] is the byte where token k starts."""
        b = self._bytes(text)
        ids, spans, _ = self.encode_batch_spans(b, [0, len(b)])
        return ids, spans

    def encode_added(self, text, literals) -> np.ndarray:
        """Encode with added-token literals: literals is a list of (bytes, id); the leftmost,
        longest literal is taken at each position and the text between literals is encoded
        segment by segment."""
        b = self._bytes(text)
        blob = b"".join(x for x, _ in literals)
        off = np.cumsum([0] + [len(x) for x, _ in literals]).astype(np.uint64)
        lid = np.asarray([i for _, i in literals] or [0], dtype=np.int32)
        out = np.zeros(max(len(b), 1), dtype=np.int32)
        n = ctypes.c_size_t(0)
        rc = lib().orc_encode_added(self._h, blob, off.ctypes.data, len(literals), lid.ctypes.data, b, len(b),
                                    out.ctypes.data, out.size, ctypes.byref(n))
        if rc == 1:
            raise UnicodeDecodeError("utf-8", b, 0, len(b), "invalid UTF-8 (oracle)")
        if rc:
            raise OracleError(f"encode_added failed (code {rc})")
        return out[: n.value].copy()
