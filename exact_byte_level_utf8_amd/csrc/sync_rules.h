// Synchronizing transitions: the stable pre-tokenization boundaries that
// certify an append-repair splice (TokTier, section 3, windowed repair with a
// splice certificate, and Appendix A, Definition A.4, Theorem A.5,
// Corollary A.6).
//
// A byte b where the class changes between the code point x before b and y
// at b is synchronizing when, for every left context, the pieces from b on
// are the pieces of the text from b alone, b starts a piece, and the pieces
// before b do not depend on anything after y.  Then the stored pieces before
// b are those of the extended text, and a window's pieces from b on are too.
// The sets follow from the two pattern families (they leave out exactly the
// transitions where a character before b can join the piece at b, or the
// piece before b can take characters from b on); the tests derive them
// independently by brute force from the CPU oracle's matcher.
//
//   GPT-2 style: every class change, except after U+0020 (the optional space
//   joins the next run) and apostrophe -> s t r v m l d (a contraction may
//   begin there; the match is case-sensitive).
//   Llama-3 style: every class change, except whitespace -> letter unless the
//   whitespace is CR or LF (one non-CR/LF char prefixes a letter run),
//   U+0020 -> other (the optional space), other -> letter (one other char
//   prefixes a letter run, or a contraction), and other -> CR/LF (the other
//   piece takes trailing CR/LF).
//
//   Case-splitting (o200k-style) family, over letter-case classes (U upper or
//   title case, D lower case, C caseless letters, M marks, N, W, O): a number
//   after anything else, and from a number to anything else; a letter before
//   whitespace, before an other char that is not the apostrophe (which may
//   begin a contraction suffix), and D -> U (the case boundary) except inside
//   a mixed-case contraction suffix ('rE 'vE 'lL); a mark or an
//   other char before whitespace that is not CR/LF (an other-run may take
//   marks and trailing CR/LF); CR/LF before a letter or mark; and whitespace
//   before an other char unless the whitespace is U+0020.
//
// Per-code-point logic only, for the host repair, the device repair and the
// segment pre-tokenizer of the case-splitting family.
#pragma once

#include <stdint.h>

#ifndef TOK_HD
#define TOK_HD __host__ __device__
#endif

namespace tok {

// x, y: code points before and at the byte; cx, cy: their classes (L=0 N=1
// W=2 O=3); gpt2: the GPT-2 style family (else the Llama-3 style).
TOK_HD inline bool sync_transition_of(bool gpt2, uint32_t x, uint32_t cx, uint32_t y, uint32_t cy) {
  if (cx == cy) return false;
  if (gpt2) {
    if (x == 0x20) return false;
    if (x == 0x27 && (y == 's' || y == 't' || y == 'r' || y == 'v' || y == 'm' || y == 'l' || y == 'd'))
      return false;
    return true;
  }
  const bool x_crlf = x == 0x0D || x == 0x0A, y_crlf = y == 0x0D || y == 0x0A;
  if (cx == 2u && cy == 0u && !x_crlf) return false;  // W -> L
  if (x == 0x20 && cy == 3u) return false;            // space -> O
  if (cx == 3u && cy == 0u) return false;             // O -> L
  if (cx == 3u && y_crlf) return false;               // O -> CR/LF
  return true;
}

// Case-splitting family.  sx, sy: letter-case classes of x and y (U=0 D=1
// C=2 M=3 N=4 W=5 O=6).
TOK_HD inline bool sync_transition_case(uint32_t x, uint32_t sx, uint32_t y, uint32_t sy) {
  constexpr uint32_t U = 0, D = 1, M = 3, N = 4, W = 5, O = 6;
  // written as selects: the kernels evaluate it for every code point at once
  const bool x_crlf = x == 0x0D || x == 0x0A, y_crlf = y == 0x0D || y == 0x0A;
  // after a letter: whitespace; an other char unless it is the apostrophe
  // (which may begin a contraction suffix); D -> U (the case boundary),
  // unless it is the middle of a two-letter contraction suffix in mixed case
  // ('rE 'vE 'lL)
  const bool mixed_suffix = ((x == 'r' || x == 'v') && y == 'E') || (x == 'l' && y == 'L');
  const bool after_letter = sy == W || (sy == O ? y != 0x27 : (sx == D && sy == U && !mixed_suffix));
  // after a mark or an other char: whitespace that is not CR/LF
  const bool after_mo = sy == W && !y_crlf;
  // after whitespace: an other char unless the whitespace is U+0020; a
  // letter or a mark after CR/LF
  const bool after_ws = sy != W && (sy == O ? x != 0x20 : x_crlf);
  const bool by_x = sx < M ? after_letter : (sx == M || sx == O) ? after_mo : after_ws;
  // a number after anything else, and from a number to anything else
  return sy == N ? sx != N : sx == N ? true : by_x;
}

}  // namespace tok
