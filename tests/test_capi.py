"""The C-ABI library builds, loads, exports every symbol include/tok.h
declares, and validates configurations on the host (no GPU needed: every
case here fails before any device work)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import exact_byte_level_utf8_amd as tk
from tests import libs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "tok.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tok_[a-z_]+)\s*\(", src)))


def test_header_declares_binding_exports():
    assert header_functions() == sorted(tk.EXPORTS)


def test_library_exports_every_symbol():
    libs.ensure_built()
    out = subprocess.check_output(["nm", "-D", "--defined-only", tk.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    L = tk.lib()
    for f in header_functions():
        assert getattr(L, f) is not None


def _load(merges, pattern=0):
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.uint32).reshape(-1, 2))
    h = ctypes.c_void_p()
    rc = tk.lib().tok_load(m.ctypes.data if m.size else None, m.shape[0], pattern, None, ctypes.byref(h))
    return rc, h


def test_load_rejects_bad_merges_and_pattern():
    libs.ensure_built()
    # operand not yet defined: merge 0 may only use bytes
    assert _load([[256, 1]])[0] == tk.TOK_E_BADMERGES
    assert _load([[97, 98], [97, 258]])[0] == tk.TOK_E_BADMERGES
    # repeated pair
    assert _load([[97, 98], [97, 98]])[0] == tk.TOK_E_BADMERGES
    assert _load([[97, 98]], pattern=7)[0] == tk.TOK_E_PATTERN
    h = ctypes.c_void_p()
    assert tk.lib().tok_load(None, 3, 0, None, ctypes.byref(h)) == tk.TOK_E_ARG
    assert tk.lib().tok_load(None, 0, 0, None, None) == tk.TOK_E_ARG


def test_load_options():
    """tok_opts_default gives the documented defaults; an option outside its
    range is refused before any device work."""
    libs.ensure_built()
    o = tk.default_opts()
    assert (o.device, o.initial_bytes, o.repair_window, o.repair_doublings, o.repair_margin) == (0, 0, 512, 5, 8)
    m = np.asarray([[97, 98]], dtype=np.uint32)
    for field, bad in (("repair_window", 0), ("repair_window", (1 << 24) + 1), ("repair_doublings", 25),
                       ("repair_margin", (1 << 20) + 1), ("device", -1), ("initial_bytes", tk.TOK_MAX_BYTES + 1)):
        x = tk.default_opts()
        setattr(x, field, bad)
        h = ctypes.c_void_p()
        assert tk.lib().tok_load(m.ctypes.data, 1, 0, ctypes.byref(x), ctypes.byref(h)) == tk.TOK_E_ARG, field
        assert not h.value
    with pytest.raises(TypeError):
        tk.Tokenizer(m, "gpt2", bogus=1)


def test_null_arguments():
    libs.ensure_built()
    L = tk.lib()
    n = ctypes.c_size_t(5)
    assert L.tok_encode(None, None, 0, None, 0, ctypes.byref(n)) == tk.TOK_E_ARG
    assert L.tok_encode_batch(None, None, None, 0, None, 0, None) == tk.TOK_E_ARG
    assert L.tok_repair(None, None, 0, 0, None, 0, 0, ctypes.byref(n), None) == tk.TOK_E_ARG
    assert L.tok_sync_boundary(7, 97, 32) == 0  # unknown pattern
    assert L.tok_strerror(tk.TOK_E_UTF8) == b"malformed UTF-8 input"
    assert L.tok_set_graph(None, 1) == tk.TOK_E_ARG
    assert L.tok_graph_count(None) == 0
    assert L.tok_set_profiling(None, 1) == tk.TOK_E_ARG
    assert L.tok_set_added_tokens(None, None, None, 0, None) == tk.TOK_E_ARG
    assert L.tok_encode_spans(None, None, 0, None, None, 0, ctypes.byref(n)) == tk.TOK_E_ARG
    assert L.tok_encode_spans_dev(None, None, 0, None, 0, None, None, 0, None, ctypes.byref(n), None) == tk.TOK_E_ARG
    L.tok_free(None)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus 2 exits with a message and no work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_constants_match_the_header():
    """The binding's status codes and size limit are the header's #defines."""
    with open(os.path.join(ROOT, "include", "tok.h")) as f:
        text = f.read()
    defs = {m.group(1): int(m.group(2).rstrip("uUlL"), 0)
            for m in re.finditer(r"#define\s+(TOK_\w+)\s+(0x[0-9A-Fa-f]+[uUlL]*|\d+)", text)}
    for name in ("TOK_OK", "TOK_E_ARG", "TOK_E_BADMERGES", "TOK_E_PATTERN", "TOK_E_UTF8", "TOK_E_CAPACITY",
                 "TOK_E_TOOLONG", "TOK_E_DEVICE", "TOK_E_NOMEM", "TOK_E_SESSION", "TOK_MAX_BYTES",
                 "TOK_NOALLOC_MAX_BYTES"):
        assert defs[name] == getattr(tk, name), name
