// Lookahead cache (host C++): n-gram count tries per sequence and for the
// whole batch, queried by the longest matching suffix, answering with a
// best-first forest of candidates (design talk "大模型倍速推理引擎 TACO-LLM
// 的设计与实践", "1.基于批处理的 Lookahead Cache"; the readings are stated in
// pta_lookahead.h).
//
// A trie node stands for one token string p; its count is the number of
// occurrences of p.  Appending token t to a history extends every suffix of
// length < window by t, so each sequence keeps the trie nodes of its current
// suffixes (lengths 1 .. window - 1) in both tries and an append costs
// O(window) child lookups per token.  Node storage is an append-only vector,
// so node indices stay valid for the life of the cache.
#include "pta_lookahead.h"

#include <algorithm>
#include <new>
#include <queue>
#include <unordered_map>
#include <utility>
#include <vector>

namespace {

struct Trie {
  struct Node {
    int64_t count = 0;
    std::vector<std::pair<int32_t, int32_t>> kids;   // (token, node), sorted by token
  };
  std::vector<Node> nodes;
  Trie() : nodes(1) {}   // node 0: the empty string

  int32_t child(int32_t n, int32_t tok) const {
    if (n < 0) return -1;
    const auto& k = nodes[n].kids;
    auto it = std::lower_bound(k.begin(), k.end(), std::make_pair(tok, INT32_MIN));
    return it != k.end() && it->first == tok ? it->second : -1;
  }
  int32_t child_or_add(int32_t n, int32_t tok) {
    auto& k = nodes[n].kids;
    auto it = std::lower_bound(k.begin(), k.end(), std::make_pair(tok, INT32_MIN));
    if (it != k.end() && it->first == tok) return it->second;
    const int32_t id = (int32_t)nodes.size();
    k.insert(it, std::make_pair(tok, id));   // before push_back: k refers into nodes
    nodes.emplace_back();
    return id;
  }
  int64_t count(int32_t n) const { return n < 0 ? 0 : nodes[n].count; }
  // node of a token string, -1 when it never occurred
  int32_t find(const int32_t* s, int32_t len) const {
    int32_t n = 0;
    for (int32_t i = 0; i < len && n >= 0; ++i) n = child(n, s[i]);
    return n;
  }
};

struct Seq {
  std::vector<int32_t> hist;
  std::vector<int32_t> act_local, act_global;   // nodes of the suffixes of length 1, 2, ...
  Trie local;
  int32_t hit_q16 = 1 << 16;
};

// Extend every tracked suffix by tok in one trie.  act[k] is the node of the
// suffix of length k + 1, before the append and after it; the suffix of
// length window is counted but not kept (nothing extends it).  In place, from
// the longest suffix down, so each old node is read before its slot is reused.
void extend(Trie& t, std::vector<int32_t>& act, int32_t tok, int32_t window) {
  auto bump = [&](int32_t n) {
    t.nodes[n].count += 1;
    return n;
  };
  const int32_t m = (int32_t)act.size();
  if (m == window - 1)
    bump(t.child_or_add(act[m - 1], tok));
  else
    act.push_back(0);
  for (int32_t k = std::min(m, window - 2) - 1; k >= 0; --k) act[k + 1] = bump(t.child_or_add(act[k], tok));
  act[0] = bump(t.child_or_add(0, tok));
}

}  // namespace

struct taco_la_cache {
  int32_t window, max_match;
  Trie global;
  std::unordered_map<int32_t, Seq> seqs;
};

extern "C" {

taco_la_cache* taco_la_create(int32_t window, int32_t max_match) {
  if (window < 2 || window > 64 || max_match < 1 || max_match > window - 1) return nullptr;
  taco_la_cache* c = new (std::nothrow) taco_la_cache();
  if (!c) return nullptr;
  c->window = window;
  c->max_match = max_match;
  return c;
}

void taco_la_destroy(taco_la_cache* c) { delete c; }

pta_status taco_la_append(taco_la_cache* c, int32_t seq, const int32_t* tokens, int32_t n) {
  if (!c || (n > 0 && !tokens)) return PTA_ERR_NULL_PTR;
  if (seq < 0 || n < 0) return PTA_ERR_BAD_DIMS;
  for (int32_t i = 0; i < n; ++i)
    if (tokens[i] < 0) return PTA_ERR_BAD_DIMS;
  Seq& s = c->seqs[seq];
  for (int32_t i = 0; i < n; ++i) {
    s.hist.push_back(tokens[i]);
    extend(s.local, s.act_local, tokens[i], c->window);
    extend(c->global, s.act_global, tokens[i], c->window);
  }
  return PTA_OK;
}

pta_status taco_la_append_batch(taco_la_cache* c, int32_t num_seqs, const int32_t* seqs, const int32_t* lens,
                                const int32_t* tokens) {
  if (!c) return PTA_ERR_NULL_PTR;
  if (num_seqs < 0) return PTA_ERR_BAD_DIMS;
  if (num_seqs == 0) return PTA_OK;
  if (!seqs || !lens) return PTA_ERR_NULL_PTR;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (seqs[i] < 0 || lens[i] < 0) return PTA_ERR_BAD_DIMS;
    total += lens[i];
  }
  if (total > 0 && !tokens) return PTA_ERR_NULL_PTR;
  for (int64_t j = 0; j < total; ++j)
    if (tokens[j] < 0) return PTA_ERR_BAD_DIMS;
  for (int32_t i = 0; i < num_seqs; ++i) {
    taco_la_append(c, seqs[i], tokens, lens[i]);
    tokens += lens[i];
  }
  return PTA_OK;
}

pta_status taco_la_release(taco_la_cache* c, int32_t seq) {
  if (!c) return PTA_ERR_NULL_PTR;
  c->seqs.erase(seq);
  return PTA_OK;
}

pta_status taco_la_propose(taco_la_cache* c, int32_t num_seqs, const int32_t* seqs, const int32_t* budgets,
                           int32_t max_q, int32_t* tokens, int32_t* parents, int32_t* counts) {
  if (!c) return PTA_ERR_NULL_PTR;
  if (num_seqs < 0 || max_q < 1) return PTA_ERR_BAD_DIMS;
  if (num_seqs == 0) return PTA_OK;
  if (!seqs || !budgets || !tokens || !parents || !counts) return PTA_ERR_NULL_PTR;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (budgets[i] < 0 || budgets[i] > max_q) return PTA_ERR_BAD_DIMS;

  // frontier entry: a string p + x eligible as the next candidate
  struct Cand {
    int64_t score;
    int32_t parent, token, lnode, gnode;
  };
  auto worse = [](const Cand& a, const Cand& b) {   // priority: score desc, parent asc, token asc
    if (a.score != b.score) return a.score < b.score;
    if (a.parent != b.parent) return a.parent > b.parent;
    return a.token > b.token;
  };
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t* tok = tokens + (int64_t)i * max_q;
    int32_t* par = parents + (int64_t)i * max_q;
    std::fill(tok, tok + max_q, -1);
    std::fill(par, par + max_q, -1);
    counts[i] = 0;
    auto it = c->seqs.find(seqs[i]);
    if (it == c->seqs.end() || budgets[i] == 0) continue;
    const Seq& s = it->second;
    const Trie& lt = s.local;
    const Trie& gt = c->global;
    const int32_t H = (int32_t)s.hist.size();
    // longest suffix with a continuation in either cache
    int32_t ln = -1, gn = -1;
    for (int32_t k = std::min(c->max_match, H); k >= 1; --k) {
      const int32_t* suf = s.hist.data() + (H - k);
      const int32_t a = lt.find(suf, k), g = gt.find(suf, k);
      if ((a >= 0 && !lt.nodes[a].kids.empty()) || (g >= 0 && !gt.nodes[g].kids.empty())) {
        ln = a;
        gn = g;
        break;
      }
    }
    if (ln < 0 && gn < 0) continue;
    std::priority_queue<Cand, std::vector<Cand>, decltype(worse)> pq(worse);
    // the continuations of a (local, global) node pair: union of both child lists
    auto push_kids = [&](int32_t l, int32_t g, int32_t parent) {
      static const std::vector<std::pair<int32_t, int32_t>> none;
      const auto& lk = l >= 0 ? lt.nodes[l].kids : none;
      const auto& gk = g >= 0 ? gt.nodes[g].kids : none;
      size_t a = 0, b = 0;
      while (a < lk.size() || b < gk.size()) {
        int32_t t, lc = -1, gc = -1;
        if (b >= gk.size() || (a < lk.size() && lk[a].first < gk[b].first)) {
          t = lk[a].first;
          lc = lk[a++].second;
        } else if (a >= lk.size() || gk[b].first < lk[a].first) {
          t = gk[b].first;
          gc = gk[b++].second;
        } else {
          t = lk[a].first;
          lc = lk[a++].second;
          gc = gk[b++].second;
        }
        pq.push(Cand{lt.count(lc) + gt.count(gc), parent, t, lc, gc});
      }
    };
    push_kids(ln, gn, -1);
    int32_t n = 0;
    while (n < budgets[i] && !pq.empty()) {
      const Cand x = pq.top();
      pq.pop();
      tok[n] = x.token;
      par[n] = x.parent;
      push_kids(x.lnode, x.gnode, n);
      ++n;
    }
    counts[i] = n;
  }
  return PTA_OK;
}

pta_status taco_la_update_budgets(taco_la_cache* c, int32_t num_seqs, const int32_t* seqs,
                                  const int32_t* proposed, const int32_t* accepted, int32_t min_len,
                                  int32_t max_len, int32_t batch_cap, int32_t* budgets) {
  if (!c) return PTA_ERR_NULL_PTR;
  if (num_seqs < 0 || min_len < 0 || max_len < min_len || batch_cap < 0) return PTA_ERR_BAD_DIMS;
  if (num_seqs == 0) return PTA_OK;
  if (!seqs || !proposed || !accepted || !budgets) return PTA_ERR_NULL_PTR;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (proposed[i] < 0 || accepted[i] < 0 || accepted[i] > proposed[i]) return PTA_ERR_BAD_DIMS;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Seq& s = c->seqs[seqs[i]];
    if (proposed[i] > 0)
      s.hit_q16 = (int32_t)(((int64_t)s.hit_q16 + ((int64_t)accepted[i] << 16) / proposed[i]) >> 1);
    const int64_t b = ((int64_t)max_len * s.hit_q16 + (1 << 15)) >> 16;
    budgets[i] = (int32_t)std::min<int64_t>(std::max<int64_t>(b, min_len), max_len);
    total += budgets[i];
  }
  if (batch_cap > 0 && total > batch_cap)
    for (int32_t i = 0; i < num_seqs; ++i)
      budgets[i] = (int32_t)std::max<int64_t>(min_len, (int64_t)budgets[i] * batch_cap / total);
  return PTA_OK;
}

pta_status taco_la_tree_mask(int32_t num_seqs, int32_t max_q, const int32_t* parents, const int32_t* counts,
                             uint8_t* mask) {
  if (num_seqs < 0 || max_q < 1) return PTA_ERR_BAD_DIMS;
  if (num_seqs == 0) return PTA_OK;
  if (!parents || !counts || !mask) return PTA_ERR_NULL_PTR;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (counts[s] < 0 || counts[s] > max_q) return PTA_ERR_BAD_DIMS;
    const int32_t* p = parents + (int64_t)s * max_q;
    for (int32_t i = 0; i < counts[s]; ++i)
      if (p[i] < -1 || p[i] >= i) return PTA_ERR_BAD_DIMS;
  }
  const int64_t per = (int64_t)max_q * max_q;
  std::fill(mask, mask + per * num_seqs, (uint8_t)0);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t* p = parents + (int64_t)s * max_q;
    uint8_t* m = mask + per * s;
    for (int32_t i = 0; i < counts[s]; ++i)
      for (int32_t j = i; j >= 0; j = p[j]) m[(int64_t)i * max_q + j] = 1;
  }
  return PTA_OK;
}

}  // extern "C"
