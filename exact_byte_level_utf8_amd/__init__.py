"""Python binding of the HIP tokenizer library (libtok.so, include/tok.h).

Argument marshalling only: every step of the tokenizer runs in the library's
HIP kernels.  Device-pointer calls take torch tensors (used only as device
buffers) and enqueue on torch's current stream unless a stream is given.  The
library must be built first (``python -m exact_byte_level_utf8_amd.build``);
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtok.so")

PATTERNS = {"gpt2": 0, "llama3": 1, "o200k": 2}

TOK_OK, TOK_E_ARG, TOK_E_BADMERGES, TOK_E_PATTERN, TOK_E_UTF8 = 0, 1, 2, 3, 4
TOK_E_CAPACITY, TOK_E_TOOLONG, TOK_E_DEVICE, TOK_E_NOMEM, TOK_E_SESSION = 5, 6, 7, 8, 9
TOK_MAX_BYTES = 0xFFFF0000  # longest input, in bytes
TOK_NOALLOC_MAX_BYTES = 1 << 20  # longest input of tok_encode_dev_noalloc

# every function declared in include/tok.h
EXPORTS = (
    "tok_opts_default", "tok_load", "tok_free", "tok_strerror", "tok_encode", "tok_encode_dev", "tok_encode_batch",
    "tok_encode_batch_dev", "tok_encode_spans_dev", "tok_encode_spans", "tok_pretokenize_dev", "tok_repair",
    "tok_repair_dev", "tok_sync_boundary", "tok_get_info",
    "tok_token_lengths", "tok_set_added_tokens", "tok_set_graph", "tok_graph_count", "tok_set_profiling", "tok_stage_ms",
    "tok_fill_scratch", "tok_encode_dev_noalloc",
)


class TokError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_strerror(code)} (code {code})")
        self.code = code


class TokInfo(ctypes.Structure):
    _fields_ = [("pattern", ctypes.c_uint32), ("n_merges", ctypes.c_uint32),
                ("vocab_size", ctypes.c_uint32), ("max_token_len", ctypes.c_uint32),
                ("n_whole", ctypes.c_uint32), ("n_not_self", ctypes.c_uint32),
                ("config_hash", ctypes.c_uint64)]


class TokOpts(ctypes.Structure):
    """tok_opts: load options (device, initial scratch, repair window, doublings, margin, hand-over wait)."""
    _fields_ = [("device", ctypes.c_int32), ("repair_window", ctypes.c_uint32),
                ("initial_bytes", ctypes.c_uint64), ("repair_doublings", ctypes.c_uint32),
                ("repair_margin", ctypes.c_uint32), ("handoff_wait_us", ctypes.c_uint32)]


def default_opts() -> TokOpts:
    o = TokOpts()
    lib().tok_opts_default(ctypes.byref(o))
    return o


class RepairInfo(ctypes.Structure):
    _fields_ = [("window_start", ctypes.c_uint64), ("splice_byte", ctypes.c_uint64),
                ("kept", ctypes.c_uint64), ("widenings", ctypes.c_uint32), ("full", ctypes.c_uint32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run python -m exact_byte_level_utf8_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        szp = ctypes.POINTER(ctypes.c_size_t)
        L.tok_opts_default.argtypes = [ctypes.POINTER(TokOpts)]
        L.tok_opts_default.restype = None
        L.tok_load.argtypes = [vp, sz, i32, ctypes.POINTER(TokOpts), ctypes.POINTER(vp)]
        L.tok_free.argtypes = [vp]
        L.tok_free.restype = None
        L.tok_strerror.argtypes = [i32]
        L.tok_strerror.restype = ctypes.c_char_p
        L.tok_encode.argtypes = [vp, vp, sz, vp, sz, szp]
        L.tok_encode_dev.argtypes = [vp, vp, sz, vp, sz, szp, vp]
        L.tok_encode_batch.argtypes = [vp, vp, vp, sz, vp, sz, vp]
        L.tok_encode_batch_dev.argtypes = [vp, vp, sz, vp, sz, vp, sz, vp, szp, vp]
        L.tok_encode_spans_dev.argtypes = [vp, vp, sz, vp, sz, vp, vp, sz, vp, szp, vp]
        L.tok_encode_spans.argtypes = [vp, vp, sz, vp, vp, sz, szp]
        L.tok_pretokenize_dev.argtypes = [vp, vp, sz, vp, sz, vp, vp]
        L.tok_repair.argtypes = [vp, vp, sz, sz, vp, sz, sz, szp, ctypes.POINTER(RepairInfo)]
        L.tok_repair_dev.argtypes = [vp, vp, sz, sz, vp, sz, sz, szp, ctypes.POINTER(RepairInfo)]
        L.tok_sync_boundary.argtypes = [i32, ctypes.c_uint32, ctypes.c_uint32]
        L.tok_get_info.argtypes = [vp, ctypes.POINTER(TokInfo)]
        L.tok_token_lengths.argtypes = [vp, vp, sz]
        L.tok_token_lengths.restype = sz
        L.tok_set_added_tokens.argtypes = [vp, vp, vp, sz, vp]
        L.tok_set_graph.argtypes = [vp, i32]
        L.tok_graph_count.argtypes = [vp]
        L.tok_graph_count.restype = sz
        L.tok_set_profiling.argtypes = [vp, i32]
        L.tok_stage_ms.argtypes = [vp, vp, i32]
        L.tok_fill_scratch.argtypes = [vp, i32]
        L.tok_encode_dev_noalloc.argtypes = [vp, vp, sz, vp, sz, szp, vp]
        for name in ("tok_load", "tok_encode", "tok_encode_dev", "tok_encode_batch", "tok_encode_batch_dev",
                     "tok_encode_spans_dev", "tok_encode_spans", "tok_pretokenize_dev", "tok_repair",
                     "tok_repair_dev", "tok_sync_boundary", "tok_get_info", "tok_set_added_tokens",
                     "tok_set_graph", "tok_set_profiling", "tok_stage_ms", "tok_fill_scratch",
                     "tok_encode_dev_noalloc"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _strerror(code: int) -> str:
    try:
        return lib().tok_strerror(code).decode()
    except ImportError:
        return "library not loaded"


def _check(rc: int, what: str) -> None:
    if rc != TOK_OK:
        raise TokError(rc, what)


def sync_boundary(pattern: str | int, prev_cp: int, cp: int) -> bool:
    """tok_sync_boundary: is prev_cp -> cp a synchronizing transition?"""
    pat = PATTERNS[pattern] if isinstance(pattern, str) else int(pattern)
    return bool(lib().tok_sync_boundary(pat, prev_cp, cp))


_DTYPES: dict = {}  # dtype_name -> the torch dtypes it names (filled on first use)


def _dev_ptr(t, dtype_name: str, what: str) -> int:
    """Device pointer of a contiguous CUDA/HIP torch tensor of the given dtype
    (dtype_name may list alternatives separated by '|')."""
    want = _DTYPES.get(dtype_name)
    if want is None:
        import torch

        want = _DTYPES[dtype_name] = tuple(getattr(torch, d) for d in dtype_name.split("|"))
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.dtype not in want:
        raise ValueError(f"{what} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _stream_handle(stream) -> int | None:
    """The HIP stream to enqueue on: torch's current stream of the current
    device when stream is None (its raw handle, without building a Stream
    object: that costs about 2.5 us per call), else the given stream."""
    if stream is None:
        import torch

        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class Tokenizer:
    """One loaded configuration (merge list + pre-tokenizer pattern) on one GPU."""

    def __init__(self, merges, pattern: str | int, device: int = 0, **opts):
        """opts: any tok_opts field other than device (initial_bytes, repair_window,
        repair_doublings, repair_margin); the rest keep their defaults."""
        m = np.ascontiguousarray(np.asarray(merges, dtype=np.uint32).reshape(-1, 2))
        pat = PATTERNS[pattern] if isinstance(pattern, str) else int(pattern)
        o = default_opts()
        o.device = device
        for k, v in opts.items():
            if k == "device" or k not in dict(TokOpts._fields_):
                raise TypeError(f"unknown tok_opts field {k!r}")
            setattr(o, k, v)
        h = ctypes.c_void_p()
        _check(lib().tok_load(m.ctypes.data if m.size else None, m.shape[0], pat, ctypes.byref(o), ctypes.byref(h)),
               "tok_load")
        self._h = h
        self.device = device
        self.pattern = pat
        self.n_merges = m.shape[0]

    def close(self) -> None:
        h = getattr(self, "_h", None)
        if h:
            lib().tok_free(h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ----------------------------------------------------------- host memory
    def encode(self, text) -> np.ndarray:
        b = text.encode("utf-8") if isinstance(text, str) else bytes(text)
        ids = np.empty(max(len(b), 1), dtype=np.int32)
        n = ctypes.c_size_t(0)
        _check(lib().tok_encode(self._h, b, len(b), ids.ctypes.data, ids.size, ctypes.byref(n)), "tok_encode")
        return ids[: n.value].copy()

    def encode_spans(self, text) -> tuple[np.ndarray, np.ndarray]:
        """tok_encode_spans: (ids, spans), spans[k] = byte where token k starts."""
        b = text.encode("utf-8") if isinstance(text, str) else bytes(text)
        ids = np.empty(max(len(b), 1), dtype=np.int32)
        spans = np.empty(max(len(b), 1), dtype=np.uint32)
        n = ctypes.c_size_t(0)
        _check(lib().tok_encode_spans(self._h, b, len(b), ids.ctypes.data, spans.ctypes.data, ids.size,
                                      ctypes.byref(n)), "tok_encode_spans")
        return ids[: n.value].copy(), spans[: n.value].copy()

    def encode_batch(self, data: bytes, doc_off) -> tuple[np.ndarray, np.ndarray]:
        off = np.ascontiguousarray(np.asarray(doc_off, dtype=np.uint64))
        n_docs = off.size - 1
        ids = np.empty(max(len(data), 1), dtype=np.int32)
        out_off = np.zeros(n_docs + 1, dtype=np.uint64)
        _check(lib().tok_encode_batch(self._h, data, off.ctypes.data, n_docs, ids.ctypes.data, ids.size,
                                      out_off.ctypes.data), "tok_encode_batch")
        return ids[: int(out_off[-1])].copy(), out_off

    def repair(self, session_ids, text: bytes, old_len: int) -> tuple[np.ndarray, dict]:
        """tok_repair: IDs of ``text`` from the IDs of ``text[:old_len]``.

        Returns (ids, info); the input array is not modified (the splice happens
        in a copy of it).
        """
        b = bytes(text)
        sess = np.asarray(session_ids, dtype=np.int32)
        cap = sess.size + (len(b) - old_len) + 64
        while True:
            buf = np.zeros(max(cap, 1), dtype=np.int32)
            buf[: sess.size] = sess
            n = ctypes.c_size_t(0)
            info = RepairInfo()
            rc = lib().tok_repair(self._h, buf.ctypes.data, sess.size, buf.size, b, old_len, len(b),
                                  ctypes.byref(n), ctypes.byref(info))
            if rc == TOK_E_CAPACITY and n.value > cap:
                cap = n.value
                continue
            _check(rc, "tok_repair")
            return buf[: n.value].copy(), {f: getattr(info, f) for f, _ in RepairInfo._fields_}

    def repair_into(self, buf: np.ndarray, n_session: int, text: bytes, old_len: int) -> tuple[int, dict]:
        """tok_repair in place on a caller-owned int32 buffer: buf[:n_session] holds the IDs of
        text[:old_len]; on return buf[:n] holds the IDs of text.  Returns (n, info)."""
        if buf.dtype != np.int32 or not buf.flags.c_contiguous:
            raise ValueError("buf must be a contiguous int32 array")
        n = ctypes.c_size_t(0)
        info = RepairInfo()
        _check(lib().tok_repair(self._h, buf.ctypes.data, n_session, buf.size, text, old_len, len(text),
                                ctypes.byref(n), ctypes.byref(info)), "tok_repair")
        return n.value, {f: getattr(info, f) for f, _ in RepairInfo._fields_}

    def repair_dev(self, d_session, n_session: int, text: bytes, old_len: int) -> tuple[int, dict]:
        """tok_repair_dev: d_session (int32 device tensor, its size is the capacity) holds the IDs of
        text[:old_len] in its first n_session entries; on return the first n hold the IDs of text.
        Returns (n, info)."""
        n = ctypes.c_size_t(0)
        info = RepairInfo()
        _check(lib().tok_repair_dev(self._h, _dev_ptr(d_session, "int32", "session"), n_session,
                                    d_session.numel(), text, old_len, len(text), ctypes.byref(n),
                                    ctypes.byref(info)), "tok_repair_dev")
        return n.value, {f: getattr(info, f) for f, _ in RepairInfo._fields_}

    # --------------------------------------------------------- device memory
    def encode_dev(self, d_text, d_ids, length: int | None = None, stream=None) -> int:
        """Encode d_text[:length] (uint8 device tensor) into d_ids (int32); returns the count."""
        n_bytes = d_text.numel() if length is None else int(length)
        n = ctypes.c_size_t(0)
        _check(lib().tok_encode_dev(self._h, _dev_ptr(d_text, "uint8", "text"), n_bytes,
                                    _dev_ptr(d_ids, "int32", "ids"), d_ids.numel(), ctypes.byref(n),
                                    _stream_handle(stream)), "tok_encode_dev")
        return n.value

    def encode_dev_noalloc(self, d_text, d_ids, length: int | None = None, stream=None) -> int:
        """tok_encode_dev_noalloc: as encode_dev, with no allocation during the call (inputs up to
        TOK_NOALLOC_MAX_BYTES)."""
        n_bytes = d_text.numel() if length is None else int(length)
        n = ctypes.c_size_t(0)
        _check(lib().tok_encode_dev_noalloc(self._h, _dev_ptr(d_text, "uint8", "text"), n_bytes,
                                            _dev_ptr(d_ids, "int32", "ids"), d_ids.numel(), ctypes.byref(n),
                                            _stream_handle(stream)), "tok_encode_dev_noalloc")
        return n.value

    def encode_batch_dev(self, d_text, d_doc_off, d_ids, d_out_off, stream=None) -> int:
        n = ctypes.c_size_t(0)
        _check(lib().tok_encode_batch_dev(self._h, _dev_ptr(d_text, "uint8", "text"), d_text.numel(),
                                          _dev_ptr(d_doc_off, "uint64", "doc_off"), d_doc_off.numel() - 1,
                                          _dev_ptr(d_ids, "int32", "ids"), d_ids.numel(),
                                          _dev_ptr(d_out_off, "uint64", "out_off"), ctypes.byref(n),
                                          _stream_handle(stream)), "tok_encode_batch_dev")
        return n.value

    def encode_spans_dev(self, d_text, d_ids, d_spans, d_doc_off=None, d_out_off=None, length: int | None = None,
                         stream=None) -> int:
        """tok_encode_spans_dev: IDs into d_ids (int32) and each token's first byte into d_spans
        (uint32 tensor, or int32 holding uint32 offsets); with d_doc_off (uint64) a batch, whose
        per-document output offsets go to d_out_off (uint64).  Returns the count."""
        n_bytes = d_text.numel() if length is None else int(length)
        if d_spans.numel() < d_ids.numel():
            raise ValueError("spans must hold as many entries as ids")
        doc = _dev_ptr(d_doc_off, "uint64", "doc_off") if d_doc_off is not None else None
        n_docs = d_doc_off.numel() - 1 if d_doc_off is not None else 0
        oo = _dev_ptr(d_out_off, "uint64", "out_off") if d_out_off is not None else None
        n = ctypes.c_size_t(0)
        _check(lib().tok_encode_spans_dev(self._h, _dev_ptr(d_text, "uint8", "text"), n_bytes, doc, n_docs,
                                          _dev_ptr(d_ids, "int32", "ids"), _dev_ptr(d_spans, "int32|uint32", "spans"),
                                          d_ids.numel(), oo, ctypes.byref(n), _stream_handle(stream)),
               "tok_encode_spans_dev")
        return n.value

    def pretokenize_dev(self, d_text, d_flags, d_doc_off=None, stream=None) -> None:
        """Piece-start flag words (uint16 per 16 bytes) of d_text into d_flags."""
        doc = _dev_ptr(d_doc_off, "uint64", "doc_off") if d_doc_off is not None else None
        n_docs = d_doc_off.numel() - 1 if d_doc_off is not None else 0
        _check(lib().tok_pretokenize_dev(self._h, _dev_ptr(d_text, "uint8", "text"), d_text.numel(), doc,
                                         n_docs, _dev_ptr(d_flags, "int16", "flags"), _stream_handle(stream)),
               "tok_pretokenize_dev")

    # ---------------------------------------------------------------- facts
    def info(self) -> dict:
        i = TokInfo()
        _check(lib().tok_get_info(self._h, ctypes.byref(i)), "tok_get_info")
        return {f: getattr(i, f) for f, _ in TokInfo._fields_}

    def token_lengths(self) -> np.ndarray:
        v = lib().tok_token_lengths(self._h, None, 0)
        out = np.zeros(v, dtype=np.uint32)
        lib().tok_token_lengths(self._h, out.ctypes.data, v)
        return out

    def set_added_tokens(self, literals) -> None:
        """tok_set_added_tokens: literals is a list of (bytes or str, id); [] removes them."""
        lits = [(x.encode("utf-8") if isinstance(x, str) else bytes(x), int(i)) for x, i in literals]
        blob = b"".join(x for x, _ in lits)
        off = np.cumsum([0] + [len(x) for x, _ in lits]).astype(np.uint64)
        ids = np.asarray([i for _, i in lits] or [0], dtype=np.int32)
        _check(lib().tok_set_added_tokens(self._h, blob if lits else None, off.ctypes.data if lits else None,
                                          len(lits), ids.ctypes.data if lits else None), "tok_set_added_tokens")

    def fill_scratch(self, value: int) -> None:
        """tok_fill_scratch: poison the context's per-call device buffers (a diagnostic)."""
        _check(lib().tok_fill_scratch(self._h, int(value)), "tok_fill_scratch")

    def set_graph(self, on: bool = True) -> None:
        """Replay a captured HIP graph for call shapes met before (tok_set_graph)."""
        _check(lib().tok_set_graph(self._h, 1 if on else 0), "tok_set_graph")

    def graph_count(self) -> int:
        return int(lib().tok_graph_count(self._h))

    def set_profiling(self, stages=True) -> None:
        """stages: True for every stage, False for none, or a bit mask (bit i = STAGES[i])."""
        mask = (1 << len(STAGES)) - 1 if stages is True else 0 if stages is False else int(stages)
        _check(lib().tok_set_profiling(self._h, mask), "tok_set_profiling")

    def stage_ms(self) -> list[float]:
        out = (ctypes.c_float * len(STAGES))()
        k = lib().tok_stage_ms(self._h, out, len(STAGES))
        return list(out[:k])


STAGES = ("pretokenize", "pieces", "assemble")


def flags_to_starts(flags: np.ndarray, n: int) -> np.ndarray:
    """Byte offsets of the set bits of piece-start flag words (uint16 per 16 bytes)."""
    w = np.asarray(flags, dtype=np.uint16)
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    return np.flatnonzero(bits[:n]).astype(np.uint64)
