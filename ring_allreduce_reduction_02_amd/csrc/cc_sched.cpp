// Host-side builders of the descriptor-step AllReduce schedules.
//
// Each builder walks the schedule's steps once and records two things: the
// descriptors the step kernel executes (combines into partials, the final
// rounded result, copies of finished values), and the transfers the
// simulated network carries (values sent per rank, number of steps), which
// cc_get_traffic reports.  Where a step's combine needs a partial that a rank
// "receives", the kernel reads it from the sending rank's partial buffer:
// every rank of one GPU sees every buffer.
#include "cc_sched.h"

#include <algorithm>

namespace cc {

namespace {

struct Builder {
  int N;
  uint64_t M;
  Plan p;
  std::vector<GDesc> cur;

  Builder(int n, uint64_t m) : N(n), M(m) { p.sent.assign(n, 0); }
  void add(const GDesc& d) {
    if (d.len) cur.push_back(d);
  }
  void flush() {
    p.steps.push_back(cur);
    cur.clear();
  }
  void send(int r, uint64_t n) { p.sent[r] += n; }
};

GDesc combine(uint64_t lo, uint64_t len, int dst, bool local_send, int in1, bool in1_send, int in2 = -1,
              bool in2_send = false, bool final_ = false) {
  GDesc d{lo, len, dst, in1, in2 < 0 ? 0 : in2, 0u};
  if (local_send) d.flags |= GD_LOCAL_SEND;
  if (in1 >= 0) d.flags |= GD_IN1 | (in1_send ? GD_IN1_SEND : 0u);
  if (in1 < 0) d.in1 = 0;
  if (in2 >= 0) d.flags |= GD_IN2 | (in2_send ? GD_IN2_SEND : 0u);
  if (final_) d.flags |= GD_FINAL;
  return d;
}

GDesc copy(uint64_t lo, uint64_t len, int dst, int src) { return GDesc{lo, len, dst, src, 0, GD_COPY}; }

uint64_t bound(uint64_t M, int parts, int c) { return (uint64_t)(((unsigned __int128)c * M) / (unsigned)parts); }

int md(int x, int n) { return ((x % n) + n) % n; }

// Binomial tree (textbook ch. 6, "Tree AllReduce"): at distance d = 1, 2, 4
// ... rank i with i mod 2d = d sends its partial to i - d, which folds
// op(own, incoming); rank 0 rounds once and the result doubles back down.
Plan tree(int N, uint64_t M) {
  Builder b(N, M);
  std::vector<char> touched(N, 0);
  int d = 1;
  for (; d < N; d *= 2) {
    const bool last = 2 * d >= N;
    for (int i = d; i < N; i += 2 * d) {
      b.add(combine(0, M, i - d, !touched[i - d], i, !touched[i], -1, false, last));
      touched[i - d] = 1;
      b.send(i, M);
    }
    b.flush();
  }
  for (d /= 2; d >= 1; d /= 2) {
    for (int i = 0; i + d < N; i += 2 * d) {
      b.add(copy(0, M, i + d, i));
      b.send(i, M);
    }
    b.flush();
  }
  b.p.net_steps = (int)b.p.steps.size();
  return b.p;
}

int height(const std::vector<std::vector<int>>& ch, int x, std::vector<int>& h) {
  if (h[x] >= 0) return h[x];
  int v = 0;
  for (int y : ch[x]) v = std::max(v, 1 + height(ch, y, h));
  return h[x] = v;
}

// Double binary tree (AllReduce notes, 算法三): elements [0, M/2) reduce and
// broadcast on T1, the rest on T2, both trees in the same steps.  A node
// combines op(op(own, left), right) in the step after its children's
// subtrees are complete; the tops round once; broadcast copies go down one
// level per step.
Plan dbt(int N, uint64_t M) {
  Builder b(N, M);
  const Trees t = dbt_trees(N);
  const uint64_t h = M / 2;
  const uint64_t lo[2] = {0, h}, len[2] = {h, M - h};
  std::vector<int> ht[2], dep[2];
  int H = 0;
  for (int k = 0; k < 2; ++k) {
    ht[k].assign(N, -1);
    H = std::max(H, height(t.ch[k], t.top[k], ht[k]));
    dep[k].assign(N, 0);
    std::vector<int> todo{t.top[k]};
    while (!todo.empty()) {
      const int x = todo.back();
      todo.pop_back();
      for (int y : t.ch[k][x]) {
        dep[k][y] = dep[k][x] + 1;
        todo.push_back(y);
      }
    }
  }
  // network: at step s the nodes of height s send their partial up
  // kernels: at step s the nodes of height s+1 fold their children in
  for (int s = 0; s < H; ++s) {
    for (int k = 0; k < 2; ++k)
      for (int x = 0; x < N; ++x) {
        if (ht[k][x] == s && x != t.top[k]) b.send(x, len[k]);
        if (ht[k][x] != s + 1) continue;
        const auto& c = t.ch[k][x];
        const int l = c.size() > 0 ? c[0] : -1, r = c.size() > 1 ? c[1] : -1;
        b.add(combine(lo[k], len[k], x, true, l, l >= 0 && ht[k][l] == 0, r, r >= 0 && ht[k][r] == 0,
                      x == t.top[k]));
      }
    b.flush();
  }
  for (int s = 0; s < H; ++s) {
    for (int k = 0; k < 2; ++k)
      for (int x = 0; x < N; ++x)
        if (dep[k][x] == s)
          for (int y : t.ch[k][x]) {
            b.add(copy(lo[k], len[k], y, x));
            b.send(x, len[k]);
          }
    b.flush();
  }
  b.p.net_steps = 2 * H;
  return b.p;
}

// 2-port ring (AllReduce notes, "2-port Ring 优化"): chunk c is owned by rank
// c and reduced by a clockwise chain over ranks c-a .. c-1 and a
// counter-clockwise chain over c+b .. c+1 (a = N/2, b = (N-1)/2), each rank
// folding op(own, partial); the owner ends with op(op(x_c, cw), ccw), reading
// the counter-clockwise partial where rank c+1 left it.  The AllGather sends
// the chunk a ranks one way and b the other.
Plan ring2(int N, uint64_t M) {
  Builder b(N, M);
  const int ca = N / 2, cb = (N - 1) / 2;
  for (int s = 0; s < ca; ++s) {
    for (int c = 0; c < N; ++c) {
      const uint64_t lo = bound(M, N, c), len = bound(M, N, c + 1) - lo;
      int src = md(c - ca + s, N), dst = md(src + 1, N);
      b.send(src, len);
      if (dst != c) {
        b.add(combine(lo, len, dst, true, src, s == 0));
      } else {
        const int in2 = cb >= 1 ? md(c + 1, N) : -1;
        b.add(combine(lo, len, c, true, src, s == 0, in2, cb == 1, true));
      }
      if (s < cb) {
        src = md(c + cb - s, N);
        dst = md(src - 1, N);
        b.send(src, len);
        if (dst != c) b.add(combine(lo, len, dst, true, src, s == 0));
      }
    }
    b.flush();
  }
  for (int s = 0; s < ca; ++s) {
    for (int c = 0; c < N; ++c) {
      const uint64_t lo = bound(M, N, c), len = bound(M, N, c + 1) - lo;
      int src = md(c + s, N);
      b.add(copy(lo, len, md(src + 1, N), src));
      b.send(src, len);
      if (s < cb) {
        src = md(c - s, N);
        b.add(copy(lo, len, md(src - 1, N), src));
        b.send(src, len);
      }
    }
    b.flush();
  }
  b.p.net_steps = 2 * ca;
  return b.p;
}

// N not a power of two (AllReduce notes, 算法二 "非 2^k 处理" and 算法四; blog,
// RHD "非 2 的整数次幂场景"): ranks 2i+1 (i < r) send their vector to 2i, which
// folds op(own, incoming); the m = 2^floor(log2 N) ranks 0, 2, .., 2r-2,
// 2r, .., N-1 run the power-of-two schedule as virtual ranks; 2i copies the
// result back to 2i+1.
Plan pairs(int N, uint64_t M, bool hd) {
  Builder b(N, M);
  int m = 1;
  while (2 * m <= N) m *= 2;
  const int r = N - m;
  std::vector<int> act(m);
  for (int v = 0; v < m; ++v) act[v] = v < r ? 2 * v : v + r;
  std::vector<char> touched(N, 0);
  for (int i = 0; i < r; ++i) {
    b.add(combine(0, M, 2 * i, true, 2 * i + 1, true));
    b.send(2 * i + 1, M);
    touched[2 * i] = 1;
  }
  b.flush();
  if (hd) {
    // halving: distance m/2 first; the rank whose bit d is 0 keeps the lower
    // half of its chunk range (m chunks)
    std::vector<int> lo(m, 0), hi(m, m);
    for (int d = m / 2; d >= 1; d /= 2) {
      std::vector<int> klo(m), khi(m);
      for (int v = 0; v < m; ++v) {
        const int mid = (lo[v] + hi[v]) / 2;
        if (v & d) klo[v] = mid, khi[v] = hi[v];
        else klo[v] = lo[v], khi[v] = mid;
      }
      for (int v = 0; v < m; ++v) {
        const int p = v ^ d;
        const uint64_t e0 = bound(M, m, klo[v]), e1 = bound(M, m, khi[v]);
        b.add(combine(e0, e1 - e0, act[v], !touched[act[v]], act[p], !touched[act[p]], -1, false, d == 1));
        b.send(act[p], e1 - e0);
      }
      for (int v = 0; v < m; ++v) {
        touched[act[v]] = 1;
        lo[v] = klo[v];
        hi[v] = khi[v];
      }
      b.flush();
    }
    // doubling: partners swap the ranges they hold
    for (int d = 1; d < m; d *= 2) {
      std::vector<int> nlo(m), nhi(m);
      for (int v = 0; v < m; ++v) {
        const int p = v ^ d;
        const uint64_t e0 = bound(M, m, lo[p]), e1 = bound(M, m, hi[p]);
        b.add(copy(e0, e1 - e0, act[v], act[p]));
        b.send(act[p], e1 - e0);
        nlo[v] = std::min(lo[v], lo[p]);
        nhi[v] = std::max(hi[v], hi[p]);
      }
      lo = nlo;
      hi = nhi;
      b.flush();
    }
  } else {
    // butterfly: full exchange at distance 1, 2, 4 ...; one descriptor
    // updates both partners from the same operands
    for (int k = 1; k < m; k *= 2) {
      for (int v = 0; v < m; ++v) {
        const int p = v ^ k;
        b.send(act[p], M);
        if (p < v) continue;
        GDesc g = combine(0, M, act[v], !touched[act[v]], act[p], !touched[act[p]], -1, false, 2 * k >= m);
        g.flags |= GD_BOTH;
        b.add(g);
      }
      for (int v = 0; v < m; ++v) touched[act[v]] = 1;
      b.flush();
    }
  }
  for (int i = 0; i < r; ++i) {
    b.add(copy(0, M, 2 * i + 1, 2 * i));
    b.send(2 * i, M);
  }
  b.flush();
  b.p.net_steps = (int)b.p.steps.size();
  return b.p;
}

}  // namespace

void hier_levels(const std::vector<int>& dims, std::vector<int>* p, std::vector<int>* stride) {
  p->clear();
  stride->clear();
  int st = 1;
  for (int q : dims) {
    if (q > 1) {
      p->push_back(q);
      stride->push_back(st);
    }
    st *= q;
  }
}

// Multi-dimensional AllReduce (AllReduce notes, 算法五; textbook ch. 6,
// "分层全归约"), one ring step per kernel step, all groups of a level side by
// side.  At an inner level the member at coordinate k receives, at ring step
// s, chunk (k-s-2) mod p of the group's range from member k-1 and folds
// op(own, incoming) -- the standalone ReduceScatter, after which member c
// holds chunk c; "own" is the rank's send buffer at the first level it takes
// part in and its partial after that.  The outermost level runs the ring
// AllReduce (chunk (k-s-1) at step s, member k then holding chunk k+1, the
// last fold written rounded to recv), its AllGather, and the inner levels'
// AllGathers copy finished ranges back out.
Plan build_hier_plan(const std::vector<int>& dims, uint64_t M) {
  std::vector<int> p, stride;
  hier_levels(dims, &p, &stride);
  int N = 1;
  for (int q : dims) N *= q;
  Builder b(N, M);
  const int d = (int)p.size();
  b.p.level_sent.assign(d, std::vector<uint64_t>(N, 0));
  std::vector<uint64_t> lo(N, 0), hi(N, M);
  auto groups = [&](int i) {
    std::vector<std::vector<int>> g;
    for (int r = 0; r < N; ++r)
      if ((r / stride[i]) % p[i] == 0) {
        std::vector<int> m(p[i]);
        for (int k = 0; k < p[i]; ++k) m[k] = r + k * stride[i];
        g.push_back(m);
      }
    return g;
  };
  auto piece = [&](int r, int parts, int c, uint64_t* a, uint64_t* len) {
    const uint64_t span = hi[r] - lo[r];
    *a = lo[r] + bound(span, parts, c);
    *len = bound(span, parts, c + 1) - bound(span, parts, c);
  };
  auto send_at = [&](int level, int r, uint64_t n) {
    b.send(r, n);
    b.p.level_sent[level][r] += n;
  };
  // ReduceScatter (off = -1 inner, 0 outermost) of one level
  auto reduce_scatter = [&](int i, int off, bool last_final) {
    const auto gs = groups(i);
    const int q = p[i];
    for (int s = 0; s < q - 1; ++s) {
      for (const auto& g : gs)
        for (int k = 0; k < q; ++k) {
          const int m = g[k], snd = g[(k - 1 + q) % q];
          const int ci = md(k - s - 1 + off, q);
          uint64_t a, len;
          piece(m, q, ci, &a, &len);
          b.add(combine(a, len, m, i == 0, snd, i == 0 && s == 0, -1, false, last_final && s == q - 2));
          send_at(i, snd, len);
        }
      b.flush();
    }
  };
  auto all_gather = [&](int i, bool ar_owners) {
    const auto gs = groups(i);
    const int q = p[i];
    for (int s = 0; s < q - 1; ++s) {
      for (const auto& g : gs)
        for (int k = 0; k < q; ++k) {
          const int c = md((ar_owners ? k + 1 : k) - s, q);
          uint64_t a, len;
          piece(g[k], q, c, &a, &len);
          b.add(copy(a, len, g[(k + 1) % q], g[k]));
          send_at(i, g[k], len);
        }
      b.flush();
    }
  };
  // the outermost level of the hierarchy runs the AllReduce; when it has
  // size 1 every non-trivial level is an inner one, and the last
  // ReduceScatter writes the finished values
  const bool top = dims.back() > 1;
  const int inner = top ? d - 1 : d;
  for (int i = 0; i < inner; ++i) {
    reduce_scatter(i, -1, !top && i == inner - 1);
    for (const auto& g : groups(i))
      for (int k = 0; k < p[i]; ++k) {
        uint64_t a, len;
        piece(g[k], p[i], k, &a, &len);
        lo[g[k]] = a;
        hi[g[k]] = a + len;
      }
  }
  if (top) {
    reduce_scatter(d - 1, 0, true);
    all_gather(d - 1, true);
  }
  for (int i = inner - 1; i >= 0; --i) {
    for (const auto& g : groups(i)) {
      uint64_t l = lo[g[0]], h = hi[g[0]];
      for (int m : g) {
        l = std::min(l, lo[m]);
        h = std::max(h, hi[m]);
      }
      for (int m : g) {
        lo[m] = l;
        hi[m] = h;
      }
    }
    all_gather(i, false);
  }
  b.p.net_steps = (int)b.p.steps.size();
  return b.p;
}

// T1: the in-order binary tree over ranks 1..N-1 (x with lowest set bit b
// has the left child x - b/2 and the right child x + c, c the largest of
// b/2, b/4, ... with x + c < N), rooted at the largest power of two below N,
// with rank 0 above the root; T2: T1 with every rank x renamed x+1 mod N.
Trees dbt_trees(int N) {
  Trees t;
  t.ch[0].assign(N, {});
  if (N >= 2) {
    int root = 1;
    while (2 * root <= N - 1) root *= 2;
    t.ch[0][0].push_back(root);
    for (int x = 1; x < N; ++x) {
      const int bl = x & -x;
      if (bl < 2) continue;
      t.ch[0][x].push_back(x - bl / 2);
      int c = bl / 2;
      while (c >= 1 && x + c >= N) c /= 2;
      if (c >= 1) t.ch[0][x].push_back(x + c);
    }
  }
  t.ch[1].assign(N, {});
  for (int x = 0; x < N; ++x)
    for (int y : t.ch[0][x]) t.ch[1][(x + 1) % N].push_back((y + 1) % N);
  t.top[0] = 0;
  t.top[1] = 1 % N;
  return t;
}

Plan build_plan(SchedAlg alg, int N, uint64_t M) {
  switch (alg) {
    case SCHED_TREE: return tree(N, M);
    case SCHED_DBT: return dbt(N, M);
    case SCHED_RING2: return ring2(N, M);
    case SCHED_HD_PAIRS: return pairs(N, M, true);
    case SCHED_BFLY_PAIRS: return pairs(N, M, false);
  }
  return Plan{};
}

}  // namespace cc
