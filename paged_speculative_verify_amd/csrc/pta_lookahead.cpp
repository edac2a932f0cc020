// Lookahead cache (host C++): n-gram count tries per sequence and for the
// whole batch, queried by the longest matching suffix, answering with a
// best-first forest of candidates (design talk "大模型倍速推理引擎 TACO-LLM
// 的设计与实践", "1.基于批处理的 Lookahead Cache"; the readings are stated in
// pta_lookahead.h).
//
// A trie node stands for one token string p; its count is the number of
// occurrences of p.  Each sequence keeps, for every start position p of its
// last window - 1 tokens, the node of the string hist[p .. H - 1] in its own
// trie and in the global one (a ring of 64 slots indexed by p mod 64), so an
// append walks each tracked string down by the new tokens, O(window) child
// lookups per token, and a query finds the node of each suffix in the ring
// without searching.  Nodes are stored in blocks that never move, so node
// indices and child-list pointers stay valid for the life of the cache.
//
// Threads: the global trie is split into shards by the first token of the
// string (every extension of a string keeps its first token, so a string and
// all its continuations live in one shard).  An append batch runs one task per
// shard (the global strings starting in it, over every sequence) and one per
// sequence (its local trie); a query batch runs one task per sequence.  Tasks
// write disjoint nodes and ring slots, and the counts do not depend on the
// order of the walks, so results are the same for every thread count.
#include "pta_lookahead.h"

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <new>
#include <queue>
#include <system_error>
#include <thread>
#include <unistd.h>
#include <unordered_map>
#include <utility>
#include <vector>

namespace {

constexpr int kRing = 64;      // ring slots per sequence and trie (window <= 64)
constexpr int kShards = 64;    // global trie shards: string starting with token t -> shard t % kShards

// Node and child storage in fixed blocks that never move once allocated:
// growth copies nothing (no pause of a task while a large array is copied),
// and child lists are found through plain pointers.
struct Trie {
  using Kid = std::pair<int32_t, int32_t>;   // (token, node)
  struct Node {
    int64_t count = 0;
    int32_t n = 0, cap = 0;   // children; capacity of the child list once there are two or more
    union {
      Kid one;     // n == 1: the child itself
      Kid* many;   // n >= 2: the child list, sorted by token
    };
    Node() : one(0, 0) {}
  };
  static constexpr int kNodeShift = 10;           // 1024 nodes per block
  static constexpr int64_t kKidBlock = 1 << 12;   // child-list slots per block
  std::vector<std::unique_ptr<Node[]>> blocks;
  int32_t size = 0;
  std::vector<std::unique_ptr<Kid[]>> kid_blocks;
  Kid* kid_cur = nullptr;         // the block short lists are taken from
  int64_t kid_used = kKidBlock;   // its slots taken

  Trie() { add(); }   // node 0: the empty string

  Node& node(int32_t id) { return blocks[id >> kNodeShift][id & ((1 << kNodeShift) - 1)]; }
  const Node& node(int32_t id) const { return blocks[id >> kNodeShift][id & ((1 << kNodeShift) - 1)]; }
  int32_t add() {
    if ((size & ((1 << kNodeShift) - 1)) == 0) blocks.emplace_back(new Node[1 << kNodeShift]);
    return size++;
  }
  Kid* alloc_kids(int32_t cap) {
    if (cap > kKidBlock / 4) {   // a long list gets a block of its own
      kid_blocks.emplace_back(new Kid[cap]);
      return kid_blocks.back().get();
    }
    if (kid_used + cap > kKidBlock) {
      kid_blocks.emplace_back(new Kid[kKidBlock]);
      kid_cur = kid_blocks.back().get();
      kid_used = 0;
    }
    Kid* k = kid_cur + kid_used;
    kid_used += cap;
    return k;
  }

  // children of node x, sorted by token (a node's only child is kept in the
  // node itself, so the walks down the deep, single-child part of a trie read
  // one node per step)
  static const Kid* kids(const Node& x) { return x.n == 1 ? &x.one : x.many; }

  int32_t child_or_add(int32_t n, int32_t tok) {
    Node& x = node(n);
    const Kid* k = kids(x);
    const Kid* it = std::lower_bound(k, k + x.n, Kid(tok, INT32_MIN));
    if (it != k + x.n && it->first == tok) return it->second;
    const int32_t id = add();   // blocks never move: x stays valid
    if (x.n == 0) {
      x.one = Kid(tok, id);
    } else {
      const int32_t at = (int32_t)(it - k);
      if (x.n == 1 || x.n == x.cap) {   // to a larger list (the old one is left unused)
        const int32_t cap = x.n == 1 ? 4 : 2 * x.cap;
        Kid* m = alloc_kids(cap);
        std::copy(k, k + x.n, m);
        x.many = m;
        x.cap = cap;
      }
      std::copy_backward(x.many + at, x.many + x.n, x.many + x.n + 1);
      x.many[at] = Kid(tok, id);
    }
    x.n += 1;
    return id;
  }
  int64_t count(int32_t n) const { return n < 0 ? 0 : node(n).count; }
};

struct Seq {
  std::vector<int32_t> hist;
  int32_t hit_q16 = 1 << 16;
  int32_t cur = 0;      // which half of each ring holds the current nodes
  uint64_t epoch = 0;   // append batch that last touched the sequence
  int64_t h0 = 0;       // history length before that batch
  Trie local;
  // node of hist[p .. H - 1] in the local and the global trie at slot
  // p % kRing of half cur, for max(0, H - window + 1) <= p < H; an append
  // batch reads half cur and writes the other, so no task reads a slot
  // another task of the same batch writes
  alignas(64) int32_t lring[2][kRing];
  int32_t gring[2][kRing];
};

// One tracked string hist[p .. e - 1] being extended in an append batch: node
// is its node so far (from the ring, or the root when p >= h0), and it takes
// the tokens hist[e .. e1 - 1], counting each extension.
struct Walk {
  const int32_t* hist;
  int64_t p, e, e1;
  int32_t node;
  int32_t* out;   // the ring slot that keeps the last node, or nullptr
};

// The walk of string start p in trie ring ring[2][kRing] of sequence s, whose
// history grew from s.h0 to its current length in this batch.
Walk make_walk(const Seq& s, int64_t p, int32_t window, int32_t (*ring)[kRing]) {
  const int64_t h1 = (int64_t)s.hist.size();
  return Walk{s.hist.data(), p, std::max(p, s.h0), std::min<int64_t>(h1, p + window),
              p < s.h0 ? ring[s.cur][p % kRing] : 0,
              p + window > h1 ? &ring[s.cur ^ 1][p % kRing] : nullptr};
}

// Run the walks in rounds of one token each, so the lookups of one round are
// independent of each other (their cache misses overlap); then the strings
// still shorter than window keep their node in the ring.
void run_walks(Trie& t, std::vector<Walk>& ws) {
  for (bool more = true; more;) {
    more = false;
    for (Walk& w : ws)
      if (w.e < w.e1) {
        w.node = t.child_or_add(w.node, w.hist[w.e]);
        t.node(w.node).count += 1;
        more |= ++w.e < w.e1;
      }
  }
  for (const Walk& w : ws)
    if (w.out) *w.out = w.node;
}

// A fixed set of worker threads running one batch of tasks at a time; the
// calling thread takes part, so a pool of n threads has n - 1 workers.  A task
// is claimed by a compare-and-swap on one word that holds the batch number,
// the task count and the next task index, so a worker that wakes late for a
// finished batch claims nothing; the caller returns once every task of its
// batch is done.  Workers spin briefly for the next batch before they sleep.
class Pool {
 public:
  ~Pool() { resize(1); }
  int size() const { return orphaned() ? 1 : (int)workers_.size() + 1; }

  // false when the system refuses a thread (the pool then keeps none)
  bool resize(int n) {
    if (orphaned()) {
      // a child process after fork() has none of the parent's workers: their
      // handles are set aside unused (joining them here would wait forever)
      (void)new std::vector<std::thread>(std::move(workers_));
      workers_.clear();
    }
    if (!workers_.empty()) {
      {
        std::lock_guard<std::mutex> lk(m_);
        quit_.store(true, std::memory_order_relaxed);
        state_.store(pack(gen(state_.load(std::memory_order_relaxed)) + 1, 0, 0), std::memory_order_release);
      }
      cv_.notify_all();
      for (auto& w : workers_) w.join();
      workers_.clear();
      quit_.store(false, std::memory_order_relaxed);
    }
    // the batch number a worker starts from is taken here, not by the new
    // thread, which may first run after the next batch is published
    const uint64_t g0 = gen(state_.load(std::memory_order_acquire));
    owner_ = getpid();
    try {
      for (int i = 1; i < n; ++i) workers_.emplace_back([this, g0] { loop(g0); });
    } catch (const std::system_error&) {
      resize(1);
      return false;
    }
    return true;
  }

  // f(i) for every i in [0, count), in any order over the threads
  void run(int64_t count, const std::function<void(int64_t)>& f) {
    if (workers_.empty() || count <= 1 || orphaned()) {
      for (int64_t i = 0; i < count; ++i) f(i);
      return;
    }
    const int64_t tasks = std::min<int64_t>(count, kMaxTasks);
    const int64_t chunk = (count + tasks - 1) / tasks;
    const std::function<void(int64_t)> body = [&](int64_t t) {
      for (int64_t i = t * chunk, e = std::min(count, i + chunk); i < e; ++i) f(i);
    };
    job_ = &body;
    done_.store(0, std::memory_order_relaxed);
    uint64_t g;
    {
      std::lock_guard<std::mutex> lk(m_);
      g = (gen(state_.load(std::memory_order_relaxed)) + 1) & 0xffffff;
      state_.store(pack(g, tasks, 0), std::memory_order_release);
    }
    cv_.notify_all();
    drain(g);
    while (done_.load(std::memory_order_acquire) != tasks) relax();
    job_ = nullptr;
  }

 private:
  static constexpr int64_t kMaxTasks = (1 << 20) - 1;
  static constexpr int kSpin = 1 << 15;   // polls before a worker sleeps (about a millisecond or two)
  // a short busy-wait step that keeps the thread on its core
  static void relax() {
#if defined(__x86_64__) || defined(__i386__)
    __builtin_ia32_pause();
#else
    std::this_thread::yield();
#endif
  }
  static uint64_t pack(uint64_t g, uint64_t count, uint64_t next) {
    return (g & 0xffffff) << 40 | count << 20 | next;
  }
  static uint64_t gen(uint64_t s) { return s >> 40; }
  // the workers belong to another process (this one is a child after fork())
  bool orphaned() const { return !workers_.empty() && getpid() != owner_; }

  void drain(uint64_t g) {
    uint64_t s = state_.load(std::memory_order_acquire);
    for (;;) {
      const uint64_t count = (s >> 20) & kMaxTasks, next = s & kMaxTasks;
      if (gen(s) != g || next >= count) return;
      if (!state_.compare_exchange_weak(s, s + 1, std::memory_order_acq_rel, std::memory_order_acquire)) continue;
      (*job_)((int64_t)next);
      done_.fetch_add(1, std::memory_order_acq_rel);
      s = state_.load(std::memory_order_acquire);
    }
  }
  void loop(uint64_t seen) {
    for (;;) {
      uint64_t g = gen(state_.load(std::memory_order_acquire));
      for (int spin = 0; g == seen && spin < kSpin; ++spin) {
        relax();
        g = gen(state_.load(std::memory_order_acquire));
      }
      if (g == seen) {
        std::unique_lock<std::mutex> lk(m_);
        cv_.wait(lk, [&] { return gen(state_.load(std::memory_order_acquire)) != seen; });
        g = gen(state_.load(std::memory_order_acquire));
      }
      seen = g;
      if (quit_.load(std::memory_order_acquire)) return;
      drain(g);
    }
  }

  std::vector<std::thread> workers_;
  pid_t owner_ = 0;   // the process the workers were started in
  std::mutex m_;
  std::condition_variable cv_;
  std::atomic<uint64_t> state_{0};
  std::atomic<int64_t> done_{0};
  std::atomic<bool> quit_{false};
  const std::function<void(int64_t)>* job_ = nullptr;
};

}  // namespace

struct taco_la_cache {
  int32_t window, max_match;
  Trie global[kShards];
  std::unordered_map<int32_t, Seq> seqs;
  Pool pool;
  uint64_t epoch = 0;
  // scratch of an append batch: the sequences it touches, and the global
  // string starts (index into touched, p) sorted by shard, shard t's at
  // [shard_at[t], shard_at[t + 1])
  std::vector<Seq*> touched;
  std::vector<std::pair<int32_t, int64_t>> starts;
  int64_t shard_at[kShards + 1];
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

pta_status taco_la_set_threads(taco_la_cache* c, int32_t n) {
  if (!c) return PTA_ERR_NULL_PTR;
  if (n < 1 || n > 64) return PTA_ERR_BAD_DIMS;
  if (n == c->pool.size()) return PTA_OK;
  return c->pool.resize(n) ? PTA_OK : PTA_ERR_UNSUPPORTED;
}

int32_t taco_la_threads(const taco_la_cache* c) { return c ? c->pool.size() : 0; }

pta_status taco_la_append(taco_la_cache* c, int32_t seq, const int32_t* tokens, int32_t n) {
  if (!c || (n > 0 && !tokens)) return PTA_ERR_NULL_PTR;
  if (seq < 0 || n < 0) return PTA_ERR_BAD_DIMS;
  return taco_la_append_batch(c, 1, &seq, &n, tokens);
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

  // serial: histories grow (a sequence named twice takes both chunks in order)
  // and the global strings are listed by shard with their starting nodes
  const int32_t W = c->window;
  const uint64_t epoch = ++c->epoch;
  c->touched.clear();
  for (int32_t i = 0; i < num_seqs; ++i) {
    Seq& s = c->seqs[seqs[i]];
    if (s.epoch != epoch) {
      s.epoch = epoch;
      s.h0 = (int64_t)s.hist.size();
      c->touched.push_back(&s);
    }
    s.hist.insert(s.hist.end(), tokens, tokens + lens[i]);
    tokens += lens[i];
  }
  // the global string starts by shard (a counting sort on the first token)
  int64_t* at = c->shard_at;
  std::fill(at, at + kShards + 1, 0);
  for (Seq* s : c->touched)
    for (int64_t p = std::max<int64_t>(0, s->h0 - W + 1); p < (int64_t)s->hist.size(); ++p) ++at[s->hist[p] % kShards + 1];
  for (int t = 0; t < kShards; ++t) at[t + 1] += at[t];
  c->starts.resize(at[kShards]);
  {
    int64_t fill[kShards];
    std::copy(at, at + kShards, fill);
    for (int32_t i = 0; i < (int32_t)c->touched.size(); ++i) {
      const Seq& s = *c->touched[i];
      for (int64_t p = std::max<int64_t>(0, s.h0 - W + 1); p < (int64_t)s.hist.size(); ++p)
        c->starts[fill[s.hist[p] % kShards]++] = std::make_pair(i, p);
    }
  }

  // parallel: one task per global shard, then one per sequence's local trie
  const int64_t nt = (int64_t)c->touched.size();
  c->pool.run(kShards + nt, [&](int64_t t) {
    thread_local std::vector<Walk> ws;
    ws.clear();
    if (t < kShards) {
      for (int64_t j = at[t]; j < at[t + 1]; ++j) {
        Seq& s = *c->touched[c->starts[j].first];
        ws.push_back(make_walk(s, c->starts[j].second, W, s.gring));
      }
      run_walks(c->global[t], ws);
      return;
    }
    Seq& s = *c->touched[t - kShards];
    for (int64_t p = std::max<int64_t>(0, s.h0 - W + 1); p < (int64_t)s.hist.size(); ++p)
      ws.push_back(make_walk(s, p, W, s.lring));
    run_walks(s.local, ws);
  });
  for (Seq* s : c->touched)
    if ((int64_t)s->hist.size() > s->h0) s->cur ^= 1;
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
  struct Worse {   // priority: score desc, parent asc, token asc
    bool operator()(const Cand& a, const Cand& b) const {
      if (a.score != b.score) return a.score < b.score;
      if (a.parent != b.parent) return a.parent > b.parent;
      return a.token > b.token;
    }
  };
  c->pool.run(num_seqs, [&](int64_t i) {
    int32_t* tok = tokens + i * max_q;
    int32_t* par = parents + i * max_q;
    std::fill(tok, tok + max_q, -1);
    std::fill(par, par + max_q, -1);
    counts[i] = 0;
    auto it = c->seqs.find(seqs[i]);
    if (it == c->seqs.end() || budgets[i] == 0) return;
    const Seq& s = it->second;
    const Trie& lt = s.local;
    const int64_t H = (int64_t)s.hist.size();
    // longest suffix hist[H - k ..] with a continuation in either cache; its
    // nodes are in the rings (k <= max_match <= window - 1)
    int32_t ln = -1, gn = -1;
    const Trie* gt = nullptr;
    for (int64_t k = std::min<int64_t>(c->max_match, H); k >= 1; --k) {
      const int64_t p = H - k;
      const Trie& g = c->global[s.hist[p] % kShards];
      const int32_t a = s.lring[s.cur][p % kRing], b = s.gring[s.cur][p % kRing];
      if (lt.node(a).n > 0 || g.node(b).n > 0) {
        ln = a;
        gn = b;
        gt = &g;
        break;
      }
    }
    if (!gt) return;
    std::priority_queue<Cand, std::vector<Cand>, Worse> pq;
    // the continuations of a (local, global) node pair: union of both child lists
    auto push_kids = [&](int32_t l, int32_t g, int32_t parent) {
      const Trie::Kid* lk = l >= 0 ? Trie::kids(lt.node(l)) : nullptr;
      const Trie::Kid* gk = g >= 0 ? Trie::kids(gt->node(g)) : nullptr;
      const int32_t nl = l >= 0 ? lt.node(l).n : 0, ng = g >= 0 ? gt->node(g).n : 0;
      int32_t a = 0, b = 0;
      while (a < nl || b < ng) {
        int32_t t, lc = -1, gc = -1;
        if (b >= ng || (a < nl && lk[a].first < gk[b].first)) {
          t = lk[a].first;
          lc = lk[a++].second;
        } else if (a >= nl || gk[b].first < lk[a].first) {
          t = gk[b].first;
          gc = gk[b++].second;
        } else {
          t = lk[a].first;
          lc = lk[a++].second;
          gc = gk[b++].second;
        }
        pq.push(Cand{lt.count(lc) + gt->count(gc), parent, t, lc, gc});
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
  });
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
