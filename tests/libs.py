"""Test helpers: build-on-demand of the in-tree libraries, and the tokenizer
configurations used across the tests (merge list + pattern per config)."""
import os

import exact_byte_level_utf8_amd as tk
from exact_byte_level_utf8_amd import build as tkbuild

CONFIGS = {
    # name: (merge list, pattern)
    "tiny": ("tiny_1k", "gpt2"),
    "gpt2": ("gpt2_50k", "gpt2"),
    "llama3": ("llama3_128k", "llama3"),
    "o200k": ("o200k_64k", "o200k"),
}


def ensure_built() -> None:
    """Build libtok.so / librules_cpu.so if they are missing (never rebuilds)."""
    if not os.path.exists(tkbuild.RULES_LIB):
        tkbuild.build_rules()
    if not os.path.exists(tkbuild.LIB):
        tkbuild.build_lib()
