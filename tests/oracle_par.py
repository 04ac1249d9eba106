"""Run the CPU oracle over many documents at once, for the tests that compare
whole batches.  The oracle's ctypes calls release the GIL and share nothing
mutable, so a thread pool encodes documents in parallel; results come back in
document order."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def map_docs(fn, items) -> list:
    items = list(items)
    with ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, items))


def concat(parts) -> tuple[np.ndarray, np.ndarray]:
    """(all IDs, n_docs + 1 output offsets) of per-document ID arrays."""
    off = np.zeros(len(parts) + 1, dtype=np.uint64)
    off[1:] = np.cumsum([len(p) for p in parts])
    ids = np.concatenate([np.asarray(p, dtype=np.int32) for p in parts]) if parts else np.zeros(0, np.int32)
    return ids, off
