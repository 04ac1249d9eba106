// Deterministic greedy pair-count BPE trainer (produces the merge lists that
// serve as the frozen tokenizer configuration of every workload).
//
// Training procedure (the usual byte-level BPE training loop):
//   * the corpus arrives pre-split into pieces with their frequencies;
//   * every piece starts as its UTF-8 bytes, token IDs 0..255;
//   * repeat M times: count adjacent pairs inside pieces (weighted by piece
//     frequency), take the pair with the highest count, breaking ties by the
//     smallest (left_id, right_id) as integers; skip a pair whose concatenated
//     bytes already spell an existing token; give the merge ID 256 + r and
//     rewrite every occurrence left to right, non-overlapping;
//   * fail if the pairs run out before M merges.
//
// Usage: bpe_train <words.bin> <n_merges> <merges_out.bin>
//   words.bin : uint64 n; n x { uint64 count; uint32 len; uint8 bytes[len] }
//   merges    : n_merges x { uint32 left; uint32 right }, little endian
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <queue>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

namespace {

struct Word {
  std::vector<uint32_t> sym;
  int64_t count;
};

inline uint64_t pkey(uint32_t a, uint32_t b) { return (uint64_t(a) << 32) | b; }

struct HeapEnt {
  int64_t count;
  uint64_t key;
  bool operator<(const HeapEnt& o) const {
    // std::priority_queue pops the largest: higher count first, then the
    // smaller (left, right) pair.
    if (count != o.count) return count < o.count;
    return key > o.key;
  }
};

bool read_all(const char* path, std::vector<uint8_t>& buf) {
  FILE* f = fopen(path, "rb");
  if (!f) return false;
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  buf.resize(size_t(n));
  bool ok = fread(buf.data(), 1, buf.size(), f) == buf.size();
  fclose(f);
  return ok;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: %s words.bin n_merges merges_out.bin\n", argv[0]);
    return 2;
  }
  std::vector<uint8_t> buf;
  if (!read_all(argv[1], buf)) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 2;
  }
  const long n_merges = strtol(argv[2], nullptr, 10);
  size_t pos = 0;
  auto rd = [&](void* dst, size_t n) {
    if (pos + n > buf.size()) {
      fprintf(stderr, "truncated words file\n");
      exit(2);
    }
    memcpy(dst, buf.data() + pos, n);
    pos += n;
  };
  uint64_t n_words = 0;
  rd(&n_words, 8);
  std::vector<Word> words(n_words);
  for (uint64_t i = 0; i < n_words; ++i) {
    uint64_t c;
    uint32_t len;
    rd(&c, 8);
    rd(&len, 4);
    words[i].count = int64_t(c);
    words[i].sym.resize(len);
    for (uint32_t j = 0; j < len; ++j) words[i].sym[j] = buf[pos + j];
    pos += len;
  }

  // token strings, for the "already a token" skip
  std::vector<std::string> tok_str(256);
  std::unordered_set<std::string> tok_set;
  for (int b = 0; b < 256; ++b) {
    tok_str[b] = std::string(1, char(b));
    tok_set.insert(tok_str[b]);
  }

  std::unordered_map<uint64_t, int64_t> pair_count;
  std::unordered_map<uint64_t, std::vector<uint32_t>> where;  // may hold stale/duplicate word ids
  pair_count.reserve(1 << 22);
  where.reserve(1 << 22);
  for (uint32_t w = 0; w < n_words; ++w) {
    const auto& s = words[w].sym;
    for (size_t j = 0; j + 1 < s.size(); ++j) {
      uint64_t k = pkey(s[j], s[j + 1]);
      pair_count[k] += words[w].count;
      where[k].push_back(w);
    }
  }
  std::priority_queue<HeapEnt> heap;
  for (auto& kv : pair_count) heap.push({kv.second, kv.first});
  std::unordered_set<uint64_t> banned;

  std::vector<uint32_t> out;
  out.reserve(size_t(n_merges) * 2);
  std::vector<uint32_t> touched_words;
  std::unordered_set<uint64_t> touched_pairs;

  for (long r = 0; r < n_merges; ++r) {
    uint64_t best = 0;
    bool found = false;
    while (!heap.empty()) {
      HeapEnt e = heap.top();
      heap.pop();
      auto it = pair_count.find(e.key);
      if (it == pair_count.end() || it->second != e.count || e.count <= 0) continue;
      if (banned.count(e.key)) continue;
      uint32_t a = uint32_t(e.key >> 32), b = uint32_t(e.key & 0xffffffffu);
      std::string cat = tok_str[a] + tok_str[b];
      if (tok_set.count(cat)) {
        banned.insert(e.key);
        continue;
      }
      best = e.key;
      found = true;
      break;
    }
    if (!found) {
      fprintf(stderr, "pairs exhausted after %ld merges\n", r);
      return 3;
    }
    const uint32_t a = uint32_t(best >> 32), b = uint32_t(best & 0xffffffffu);
    const uint32_t t = 256u + uint32_t(r);
    tok_str.push_back(tok_str[a] + tok_str[b]);
    tok_set.insert(tok_str.back());
    out.push_back(a);
    out.push_back(b);

    // rewrite every word that may contain (a, b)
    std::vector<uint32_t> ws;
    ws.swap(where[best]);
    touched_pairs.clear();
    uint32_t last_w = UINT32_MAX;
    for (uint32_t w : ws) {
      if (w == last_w) continue;  // consecutive duplicates
      last_w = w;
      auto& s = words[w].sym;
      bool has = false;
      for (size_t j = 0; j + 1 < s.size(); ++j)
        if (s[j] == a && s[j + 1] == b) {
          has = true;
          break;
        }
      if (!has) continue;
      const int64_t c = words[w].count;
      for (size_t j = 0; j + 1 < s.size(); ++j) {
        uint64_t k = pkey(s[j], s[j + 1]);
        pair_count[k] -= c;
        touched_pairs.insert(k);
      }
      std::vector<uint32_t> ns;
      ns.reserve(s.size());
      for (size_t j = 0; j < s.size();) {
        if (j + 1 < s.size() && s[j] == a && s[j + 1] == b) {
          ns.push_back(t);
          j += 2;
        } else {
          ns.push_back(s[j]);
          j += 1;
        }
      }
      s.swap(ns);
      for (size_t j = 0; j + 1 < s.size(); ++j) {
        uint64_t k = pkey(s[j], s[j + 1]);
        pair_count[k] += c;
        touched_pairs.insert(k);
        if (s[j] == t || s[j + 1] == t) where[k].push_back(w);
        else if (k == best) where[k].push_back(w);
      }
    }
    for (uint64_t k : touched_pairs) {
      auto it = pair_count.find(k);
      if (it->second > 0) heap.push({it->second, k});
    }
  }

  FILE* f = fopen(argv[3], "wb");
  if (!f) {
    fprintf(stderr, "cannot write %s\n", argv[3]);
    return 2;
  }
  fwrite(out.data(), 4, out.size(), f);
  fclose(f);
  return 0;
}
