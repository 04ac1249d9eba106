"""Seeded synthetic text for the tokenizer workloads.

This module only produces text, document offsets and append splits from integer
seeds.  It holds no tokenizer arithmetic (no pre-tokenization, no BPE), so both
the CPU oracle's tests and the GPU path's tests and benchmarks may draw inputs
from it.

Workload shapes (TokTier, section 2 workload characterization and Table 2
protocol; Delta Tokenizer, section 4 setup):

* ``tiny_text``: ASCII prose from a 2,000-word Zipf(1.1) lexicon of 1-10
  letter lowercase words, with digits 0-9999, punctuation ``, . ; : ( ) '`` and
  ASCII-apostrophe contractions.
* ``mix_text``: agent-transcript-like text built from interleaved blocks of
  200-3,000 characters: English-like prose (40% of characters), code (40%) and
  pretty-printed JSON tool output (20%).  About 2% of characters are multi-byte
  UTF-8 (Latin-1 accents, CJK runs, emoji).
* ``repair_case``: a stored context plus an appended suffix whose length is
  log-normal (median 1,400 characters, clipped to [100, 20,000]); 60% of
  suffixes are tool output, and 30% start mid-word or mid-whitespace so that
  the old token boundary moves.

Lengths are in code points (characters), as the pages count them.
"""
from __future__ import annotations

import json
import math

import numpy as np

# The lexicons are fixed (independent of a text's seed), so every text of a
# workload family shares the vocabulary that its merges were trained on.
TINY_LEXICON_SEED = 1_000_003
MIX_LEXICON_SEED = 2_000_003

_LOWER = "abcdefghijklmnopqrstuvwxyz"
_CONTRACTIONS = ["s", "t", "re", "ve", "m", "ll", "d"]


def _zipf_cdf(n: int, s: float) -> np.ndarray:
    p = 1.0 / np.arange(1, n + 1, dtype=np.float64) ** s
    c = np.cumsum(p)
    return c / c[-1]


class _Sampler:
    """Bulk-buffered draws from one numpy PCG64 stream."""

    def __init__(self, seed: int):
        self.rng = np.random.default_rng(seed)
        self._u = np.empty(0)
        self._ui = 0

    def u(self) -> float:
        if self._ui >= self._u.size:
            self._u = self.rng.random(65536)
            self._ui = 0
        v = self._u[self._ui]
        self._ui += 1
        return float(v)

    def randint(self, lo: int, hi: int) -> int:
        """Uniform integer in [lo, hi]."""
        return lo + min(int(self.u() * (hi - lo + 1)), hi - lo)

    def pick(self, seq):
        return seq[min(int(self.u() * len(seq)), len(seq) - 1)]

    def zipf(self, cdf: np.ndarray) -> int:
        return min(int(np.searchsorted(cdf, self.u(), side="right")), cdf.size - 1)


# ---------------------------------------------------------------- tiny (ASCII)


def _tiny_lexicon() -> list[str]:
    rng = np.random.default_rng(TINY_LEXICON_SEED)
    words: list[str] = []
    seen = set()
    while len(words) < 2000:
        n = int(rng.integers(1, 11))
        w = "".join(_LOWER[i] for i in rng.integers(0, 26, n))
        if w not in seen:
            seen.add(w)
            words.append(w)
    return words


def tiny_text(seed: int, n_chars: int = 10_000) -> str:
    """ASCII text of exactly ``n_chars`` characters."""
    lex = _tiny_lexicon()
    cdf = _zipf_cdf(len(lex), 1.1)
    s = _Sampler(seed)
    out: list[str] = []
    total = 0
    line_left = s.randint(8, 20)
    while total < n_chars:
        if s.u() < 0.05:
            tok = str(s.randint(0, 9999))
        else:
            tok = lex[s.zipf(cdf)]
            if s.u() < 0.1:
                p = s.pick([",", ".", ";", ":", "(", ")", "'"])
                if p == "(":
                    tok = "(" + tok + ")"
                elif p == ")":
                    tok = tok + ")"
                elif p == "'":
                    tok = tok + "'" + s.pick(_CONTRACTIONS)
                else:
                    tok = tok + p
        line_left -= 1
        if line_left <= 0:
            tok += "\n"
            line_left = s.randint(8, 20)
        else:
            tok += " "
        out.append(tok)
        total += len(tok)
    return "".join(out)[:n_chars]


# ------------------------------------------------------ agent-transcript mix

_ONSETS = ["", "", "b", "c", "d", "f", "g", "h", "j", "k", "l", "m", "n", "p", "r",
           "s", "t", "v", "w", "z", "br", "ch", "cl", "dr", "fl", "gr", "pl", "pr",
           "sh", "st", "th", "tr", "qu", "sp", "wh"]
_VOWELS = ["a", "e", "i", "o", "u", "a", "e", "i", "o", "ai", "ea", "ee", "ou", "io", "y"]
_CODAS = ["", "", "", "n", "r", "s", "t", "l", "m", "nd", "st", "ng", "ck", "rt", "x"]
_ACCENTS = {"a": "áàâä", "e": "éèêë", "i": "íî", "o": "óôö", "u": "úüû", "n": "ñ", "c": "ç"}
_KEYWORDS = ["def", "return", "if", "else", "elif", "for", "while", "in", "not", "and",
             "or", "import", "from", "class", "const", "let", "var", "function", "async",
             "await", "try", "except", "catch", "finally", "with", "as", "yield", "None",
             "True", "False", "null", "self", "this", "new", "struct", "fn", "pub", "impl"]
_OPERATORS = ["=", "==", "!=", "+=", "-=", "->", "=>", "<=", ">=", "&&", "||", "+", "-",
              "*", "/", "%", "<", ">", "::", "."]
_PATH_DIRS = ["src", "lib", "tests", "app", "core", "utils", "api", "docs", "build",
              "internal", "pkg", "cmd", "tools", "data", "config"]
_EXTS = [".py", ".rs", ".ts", ".js", ".go", ".cpp", ".h", ".json", ".md", ".txt", ".yaml"]

_MIX_LEX_CACHE: list | None = None


def _mix_lexicon():
    """30,000 unique syllable-built words, ~6% carrying a Latin-1 accent."""
    global _MIX_LEX_CACHE
    if _MIX_LEX_CACHE is not None:
        return _MIX_LEX_CACHE
    s = _Sampler(MIX_LEXICON_SEED)
    words: list[str] = []
    seen = set()
    while len(words) < 30_000:
        nsyl = 1 + min(int(-math.log(1.0 - s.u()) * 1.1), 4)
        w = "".join(s.pick(_ONSETS) + s.pick(_VOWELS) + s.pick(_CODAS) for _ in range(nsyl))
        if len(w) < 2 or len(w) > 14:
            continue
        if s.u() < 0.06:
            idx = [i for i, ch in enumerate(w) if ch in _ACCENTS]
            if idx:
                i = s.pick(idx)
                w = w[:i] + s.pick(_ACCENTS[w[i]]) + w[i + 1:]
        if w not in seen:
            seen.add(w)
            words.append(w)
    _MIX_LEX_CACHE = (words, _zipf_cdf(len(words), 1.1))
    return _MIX_LEX_CACHE


class _MixGen:
    def __init__(self, seed: int):
        self.s = _Sampler(seed)
        self.words, self.cdf = _mix_lexicon()

    # -- atoms
    def word(self) -> str:
        return self.words[self.s.zipf(self.cdf)]

    def cjk(self) -> str:
        return "".join(chr(self.s.randint(0x4E00, 0x9FFF)) for _ in range(self.s.randint(2, 8)))

    def emoji(self) -> str:
        return chr(self.s.randint(0x1F300, 0x1FAFF))

    def number(self) -> str:
        u = self.s.u()
        if u < 0.6:
            return str(self.s.randint(0, 9999))
        if u < 0.8:
            return str(self.s.randint(1900, 2030))
        return f"{self.s.randint(0, 999)}.{self.s.randint(0, 99)}"

    def ident(self) -> str:
        n = self.s.randint(1, 3)
        parts = [self.word() for _ in range(n)]
        if self.s.u() < 0.55:
            return "_".join(parts)
        return parts[0] + "".join(p[:1].upper() + p[1:] for p in parts[1:])

    # -- prose
    def sentence(self) -> str:
        s = self.s
        n = s.randint(5, 20)
        toks = []
        for i in range(n):
            u = s.u()
            if u < 0.025:
                t = self.number()
            elif u < 0.045:
                t = self.cjk()
            else:
                t = self.word()
                if s.u() < 0.02:
                    t = t + "'" + s.pick(_CONTRACTIONS)
            if i == 0:
                t = t[:1].upper() + t[1:]
            if i < n - 1 and s.u() < 0.08:
                t += ","
            toks.append(t)
        end = "." if s.u() < 0.8 else s.pick(["!", "?"])
        out = " ".join(toks) + end
        if s.u() < 0.05:
            out += " " + self.emoji()
        return out

    def prose(self, target: int) -> str:
        parts = []
        total = 0
        while total < target:
            para = " ".join(self.sentence() for _ in range(self.s.randint(3, 7)))
            parts.append(para)
            total += len(para) + 2
        return "\n\n".join(parts) + "\n"

    # -- code
    def expr(self, depth: int = 0) -> str:
        s = self.s
        u = s.u()
        if u < 0.3:
            return self.ident()
        if u < 0.45:
            return self.number()
        if u < 0.6:
            q = s.pick(['"', "'"])
            body = " ".join(self.word() for _ in range(s.randint(1, 4)))
            if s.u() < 0.08:
                body = self.cjk() + " " + body
            return q + body + q
        if u < 0.8 and depth < 2:
            return self.ident() + "(" + ", ".join(self.expr(depth + 1) for _ in range(s.randint(0, 3))) + ")"
        if depth < 2:
            return self.expr(depth + 1) + " " + s.pick(_OPERATORS) + " " + self.expr(depth + 1)
        return self.ident()

    def code(self, target: int) -> str:
        s = self.s
        lines = []
        total = 0
        level = 0
        cstyle = s.u() < 0.5
        while total < target:
            ind = "    " * level
            u = s.u()
            if u < 0.08:
                line = ""
            elif u < 0.16:
                cm = "# " if not cstyle else "// "
                line = ind + cm + " ".join(self.word() for _ in range(s.randint(2, 9)))
                if s.u() < 0.15:
                    line += " " + self.cjk()
            elif u < 0.28 and level < 4:
                kw = s.pick(["def", "if", "for", "while", "function", "class", "fn"])
                head = f"{kw} {self.ident()}(" + ", ".join(self.ident() for _ in range(s.randint(0, 3))) + ")"
                line = ind + head + (" {" if cstyle else ":")
                lines.append(line)
                total += len(line) + 1
                level += 1
                continue
            elif u < 0.38 and level > 0:
                level -= 1
                line = "    " * level + ("}" if cstyle else s.pick(["pass", "return " + self.expr()]))
            elif u < 0.55:
                line = ind + "return " + self.expr() + (";" if cstyle else "")
            elif u < 0.62:
                line = ind + s.pick(_KEYWORDS) + " " + self.expr() + (";" if cstyle else "")
            else:
                op = s.pick(["=", "+=", "-=", "=", "="])
                line = ind + self.ident() + " " + op + " " + self.expr() + (";" if cstyle else "")
                if s.u() < 0.1:
                    line += " " + s.pick(["[", "{"]) + self.expr() + s.pick(["]", "}"])
            lines.append(line)
            total += len(line) + 1
        return "\n".join(lines) + "\n"

    # -- JSON tool output
    def path(self) -> str:
        s = self.s
        segs = [s.pick(_PATH_DIRS) for _ in range(s.randint(1, 4))]
        return "/" + "/".join(segs) + "/" + self.ident() + s.pick(_EXTS)

    def jvalue(self, depth: int):
        s = self.s
        u = s.u()
        if depth < 3 and u < 0.12:
            return {self.ident(): self.jvalue(depth + 1) for _ in range(s.randint(1, 5))}
        if depth < 3 and u < 0.20:
            return [self.jvalue(depth + 1) for _ in range(s.randint(1, 4))]
        u = s.u()
        if u < 0.30:
            return " ".join(self.word() for _ in range(s.randint(1, 8)))
        if u < 0.42:
            return self.path()
        if u < 0.50:
            return self.cjk() + (" " + self.word() if s.u() < 0.5 else "")
        if u < 0.65:
            return s.randint(-1000, 100000)
        if u < 0.80:
            return s.pick([-0.5, 3.14159, 1e-3, 0.25, 2.5e-07, 100.0, -12.75, 0.001, 6.02e23]) \
                if s.u() < 0.5 else round(s.u() * 1000 - 500, s.randint(1, 5))
        return s.pick([True, False, None])

    def json_block(self, target: int) -> str:
        parts = []
        total = 0
        while total < target:
            obj = {self.ident(): self.jvalue(1) for _ in range(self.s.randint(2, 8))}
            t = json.dumps(obj, indent=2, ensure_ascii=False)
            parts.append(t)
            total += len(t) + 1
        return "\n".join(parts) + "\n"

    def block(self, kind: str) -> str:
        target = self.s.randint(200, 3000)
        if kind == "prose":
            return self.prose(target)
        if kind == "code":
            return self.code(target)
        return self.json_block(target)


def mix_text(seed: int, n_chars: int) -> str:
    """Agent-transcript-like mix of exactly ``n_chars`` characters."""
    g = _MixGen(seed)
    parts: list[str] = []
    total = 0
    while total < n_chars:
        u = g.s.u()
        kind = "prose" if u < 0.4 else ("code" if u < 0.8 else "json")
        b = g.block(kind)
        parts.append(b)
        total += len(b)
    return "".join(parts)[:n_chars]


def tool_text(seed: int, n_chars: int) -> str:
    """Tool-output-only mix (code and JSON blocks) of exactly ``n_chars`` characters."""
    g = _MixGen(seed)
    parts: list[str] = []
    total = 0
    while total < n_chars:
        b = g.block("code" if g.s.u() < 0.5 else "json")
        parts.append(b)
        total += len(b)
    return "".join(parts)[:n_chars]


def prose_text(seed: int, n_chars: int) -> str:
    g = _MixGen(seed)
    parts: list[str] = []
    total = 0
    while total < n_chars:
        b = g.block("prose")
        parts.append(b)
        total += len(b)
    return "".join(parts)[:n_chars]


def chat_text(seed: int, n_chars: int, markers: list[str]) -> str:
    """Chat-transcript shape of about ``n_chars`` characters: turns of the mix
    wrapped in the given marker strings, chosen by the seed (turn open, role
    line, body, turn close).  The markers are whatever literal strings the
    caller wants to find in the text; nothing here knows what they mean."""
    g = _MixGen(seed)
    roles = ["system", "user", "assistant", "tool"]
    parts: list[str] = []
    total = 0
    while total < n_chars:
        u = g.s.u()
        kind = "prose" if u < 0.4 else ("code" if u < 0.8 else "json")
        open_m = markers[g.s.randint(0, len(markers) - 1)]
        close_m = markers[g.s.randint(0, len(markers) - 1)]
        t = open_m + roles[g.s.randint(0, 3)] + "\n" + g.block(kind) + close_m + ("\n" if g.s.u() < 0.7 else "")
        parts.append(t)
        total += len(t)
    return "".join(parts)


def cjk_text(seed: int, n_chars: int) -> str:
    """CJK-dense text of exactly ``n_chars`` characters (the CJK corpora that
    TokTier's Table 9 reports apart): runs of 50-2,000 ideographs from
    U+4E00-U+9FFF (log-uniform lengths, each character uniform as in the mix's
    CJK runs), each followed by ASCII punctuation, a newline, or a short
    phrase of lexicon words.  A run is one letter piece of up to 6,000 bytes
    under both patterns, so this text exercises the long-piece merge path."""
    g = _MixGen(seed)
    seps = [", ", ". ", ":", "! ", "? ", "\n", "\n\n", "; ", " (", ") "]
    parts: list[str] = []
    total = 0
    while total < n_chars:
        n = int(round(math.exp(math.log(50.0) + g.s.u() * (math.log(2000.0) - math.log(50.0)))))
        run = "".join(chr(g.s.randint(0x4E00, 0x9FFF)) for _ in range(n))
        u = g.s.u()
        if u < 0.7:
            tail = g.s.pick(seps)
        else:
            tail = " " + " ".join(g.word() for _ in range(g.s.randint(1, 6))) + g.s.pick(seps)
        parts.append(run + tail)
        total += len(run) + len(tail)
    return "".join(parts)[:n_chars]


# ----------------------------------------------------------------- workloads

def batch_texts(base_seed: int, n_docs: int, n_chars: int) -> list[str]:
    """``n_docs`` independent requests with per-request seeds base_seed + i."""
    return [mix_text(base_seed + i, n_chars) for i in range(n_docs)]


def pack_docs(texts: list[str]) -> tuple[bytes, np.ndarray]:
    """Concatenate UTF-8 documents; return bytes and uint64 offsets[n_docs+1]."""
    bs = [t.encode("utf-8") for t in texts]
    off = np.zeros(len(bs) + 1, dtype=np.uint64)
    off[1:] = np.cumsum([len(b) for b in bs], dtype=np.uint64)
    return b"".join(bs), off


def append_length(seed: int) -> int:
    """Log-normal append length: median 1,400 chars, sigma 1.4, clipped [100, 20000]."""
    rng = np.random.default_rng(seed)
    v = float(np.exp(math.log(1400.0) + 1.4 * rng.standard_normal()))
    return int(min(max(round(v), 100), 20_000))


def repair_case(old_seed: int, append_seed: int, old_chars: int = 1_000_000,
                append_chars: int | None = None, old_text: str | None = None):
    """Return (old_text, appended_text) for one session append.

    60% of suffixes are tool output (code/JSON), 40% prose.  30% of appends
    move the old boundary: half cut the old text inside its last letter run
    and prepend the remainder to the suffix, half end the old text in a
    newline plus spaces and start the suffix with a newline plus spaces.
    """
    old = mix_text(old_seed, old_chars) if old_text is None else old_text
    s = _Sampler(append_seed)
    n = append_length(append_seed + 7_777_777) if append_chars is None else append_chars
    if s.u() < 0.6:
        suffix = tool_text(append_seed + 1, n)
    else:
        suffix = prose_text(append_seed + 1, n)
    u = s.u()
    if u < 0.15:
        # cut inside the last letter run of the old text (needs two letters in a row)
        j = len(old) - 1
        while j > 0 and not (old[j].isalpha() and old[j - 1].isalpha()):
            j -= 1
        if j > 0:
            suffix = old[j:] + suffix
            old = old[:j]
    elif u < 0.30:
        old = old + "\n" + " " * s.randint(1, 8)
        suffix = "\n" + " " * s.randint(1, 8) + suffix
    return old, suffix
