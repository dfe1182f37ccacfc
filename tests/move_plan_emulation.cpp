// Host emulation of the handed-over compaction protocol, built with g++ from
// the same header the kernels use (kv_cache_eviction_step_amd/csrc/
// kve_move_plan.h).  Rows are tagged with the index of the token they hold;
// a step that evicted row e of n must leave rows 0 .. e-1 alone, rows
// e .. n-2 holding the old rows e+1 .. n-1, and row n-1 holding the incoming
// row (keyformer_update step 3: later rows shift down one slot, temporal
// order kept).
//
// Part 1: one cache.  For many (e, n) the step parks its rows, then the
// chunks run in random orders with their read and write phases interleaved
// at random (the move kernel gives a chunk no order with respect to another).
// Checked: no chunk reads a cache row that another chunk writes, every index
// stays inside the rows the cache holds, and the result is the shifted cache.
//
// Part 2: one launch.  Many caches reserve their chunks from one pool in a
// random order, at pool sizes from one item to more than enough.  Checked:
// accepted reservations are disjoint and inside the pool, every item the
// move kernel reads was written by this launch (an item or an empty mark),
// and every cache -- handed over or compacted in place -- ends shifted.
//
// Part 3: the pool header (counters and phase) over many calls.
//
// Exit status 0 and a summary line on success; a message and status 1 on the
// first violation.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "kve_move_plan.h"

using namespace kve;

static int fail(const char *what, int e, int n) {
  std::printf("FAIL: %s (e=%d n=%d)\n", what, e, n);
  std::exit(1);
}

struct Chunk {
  std::vector<int> vals;  // loaded source values, in destination order
  std::set<int> reads, writes;
};

// Read phase of chunk j: loads every source of its destinations.
static void chunk_read(const std::vector<int> &rows, const std::vector<int> &parked, int e, int n,
                       int j, int chunks, Chunk &c) {
  const int last = move_last_dst(n);
  const int d0 = chunk_first_dst(e, j);
  c.vals.clear();
  for (int r = 0; r < kMoveChunk; ++r) {
    const int dst = d0 + r;
    if (dst > last) break;
    const int src = chunk_source_row(e, j, chunks, dst);
    if (src < 0) {
      if (j + 1 >= chunks) fail("parked slot past the last chunk", e, n);
      c.vals.push_back(parked[j + 1]);
    } else {
      if (src < 0 || src > n - 1) fail("source row outside the cache", e, n);
      c.reads.insert(src);
      c.vals.push_back(rows[src]);
    }
    if (dst < e || dst > last) fail("destination outside the move", e, n);
    c.writes.insert(dst);
  }
  if (j == chunks - 1) c.writes.insert(n - 1);   // the incoming row
}

static void chunk_write(std::vector<int> &rows, const std::vector<int> &parked, int e, int n,
                        int j, int chunks, const Chunk &c) {
  const int d0 = chunk_first_dst(e, j);
  for (size_t r = 0; r < c.vals.size(); ++r) rows[d0 + (int)r] = c.vals[r];
  if (j == chunks - 1) rows[n - 1] = parked[0];
}

// Parks slot 0 (the incoming row) and slots 1 .. chunks-1.
static std::vector<int> park(const std::vector<int> &rows, int e, int n, int incoming) {
  const int chunks = move_chunks(e, n);
  std::vector<int> parked(chunks);
  parked[0] = incoming;
  for (int j = 1; j < chunks; ++j) {
    const int r = parked_row(e, j);
    if (r <= e || r > n - 2) fail("parked row outside the move", e, n);
    parked[j] = rows[r];
  }
  return parked;
}

static void check_shifted(const std::vector<int> &rows, int e, int n, int incoming) {
  for (int i = 0; i < e; ++i)
    if (rows[i] != i) fail("a row before the evicted one changed", e, n);
  for (int i = e; i < n - 1; ++i)
    if (rows[i] != i + 1) fail("a moved row is wrong", e, n);
  if (rows[n - 1] != incoming) fail("the incoming row is not at n-1", e, n);
}

// Runs the chunks of one handed-over move in a random interleaving.
static void run_move(std::vector<int> &rows, const std::vector<int> &parked, int e, int n,
                     std::mt19937 &rng) {
  const int chunks = move_chunks(e, n);
  std::vector<Chunk> cs(chunks);
  std::vector<int> events;                 // 2j: read of chunk j, 2j+1: its write
  for (int j = 0; j < chunks; ++j) events.push_back(2 * j);
  std::shuffle(events.begin(), events.end(), rng);
  // insert each write at a random position after its read
  std::vector<int> order;
  for (int ev : events) order.push_back(ev);
  for (int j = 0; j < chunks; ++j) {
    size_t at = 0;
    while (order[at] != 2 * j) ++at;
    std::uniform_int_distribution<size_t> pick(at + 1, order.size());
    order.insert(order.begin() + (long)pick(rng), 2 * j + 1);
  }
  for (int ev : order) {
    const int j = ev / 2;
    if (ev % 2 == 0)
      chunk_read(rows, parked, e, n, j, chunks, cs[j]);
    else
      chunk_write(rows, parked, e, n, j, chunks, cs[j]);
  }
  for (int a = 0; a < chunks; ++a)
    for (int b = 0; b < chunks; ++b)
      if (a != b)
        for (int r : cs[a].reads)
          if (cs[b].writes.count(r)) fail("a chunk reads a row another chunk writes", e, n);
}

// Part 1: every handed-over eviction of caches of n rows (a stride over e
// for the largest n), several interleavings each.
static long part1(std::mt19937 &rng) {
  long moves = 0;
  const int ns[] = {kDeferRows + 2, kDeferRows + 3, 2 * kMoveChunk + 64, 193, 200, 257, 1000,
                    1024, 1025, 2048, 4097, 6144, 12288};
  for (int n : ns) {
    const int stride = n > 4096 ? 37 : 1;
    for (int e = -1; e <= n; e += (e < 2 || e > n - kDeferRows - 4) ? 1 : stride) {
      const bool over = move_handed_over(e, n);
      // the threshold: moves of more than kDeferRows rows, interior evictions only
      if (over != (e >= 0 && e < n - 1 && n - 1 - e > kDeferRows)) fail("threshold", e, n);
      if (!over) continue;
      const int chunks = move_chunks(e, n);
      if (chunks < 2 || chunks > max_move_chunks(n)) fail("chunk count", e, n);
      if ((chunks - 1) * kMoveChunk >= n - 1 - e || chunks * kMoveChunk < n - 1 - e)
        fail("chunks do not cover the move exactly", e, n);
      for (int rep = 0; rep < (n > 2048 ? 1 : 3); ++rep) {
        std::vector<int> rows(n + 1);
        for (int i = 0; i <= n; ++i) rows[i] = i;   // row n: never read (the incoming row waits)
        rows[n] = -77;
        const std::vector<int> parked = park(rows, e, n, n);
        run_move(rows, parked, e, n, rng);
        check_shifted(rows, e, n, n);
        if (rows[n] != -77) fail("row n written", e, n);
        ++moves;
      }
    }
  }
  // the step kernel writes one item per thread of a 512-thread workgroup
  if (max_move_chunks(12288) > 512) fail("more chunks than step threads", 0, 12288);
  return moves;
}

// Part 2: one launch of many caches sharing a pool.
struct Item {
  int cache = -1;   // -1: never written; -2: marked empty
  int j = 0, base = 0;
};

static long part2(std::mt19937 &rng) {
  long launches = 0;
  const int budgets[] = {300, 1024, 6144};
  for (int budget : budgets) {
    const int caches = 64;
    const int need = caches * max_move_chunks(budget);
    for (int cap : {1, 3, 7, 40, need / 4, need}) {
      for (int rep = 0; rep < 4; ++rep) {
        std::uniform_int_distribution<int> pe(-1, budget);
        std::vector<int> es(caches);
        std::vector<std::vector<int>> rows(caches);
        for (int c = 0; c < caches; ++c) {
          es[c] = (c % 3 == 0) ? std::uniform_int_distribution<int>(0, 8)(rng) : pe(rng);
          rows[c].resize(budget + 1);
          for (int i = 0; i <= budget; ++i) rows[c][i] = i;
        }
        std::vector<Item> items(cap);
        std::vector<std::vector<int>> parked(cap);  // per item slot: the parked value
        std::vector<int> order(caches);
        for (int c = 0; c < caches; ++c) order[c] = c;
        std::shuffle(order.begin(), order.end(), rng);
        int count = 0;                                // the pool counter, zero between calls
        std::vector<std::vector<int>> cache_parked(caches);
        std::vector<bool> handed(caches, false);
        for (int c : order) {                         // the order the atomics land in
          const int e = es[c], n = budget;
          if (!move_handed_over(e, n)) continue;
          const int chunks = move_chunks(e, n);
          const int base = count;
          count += chunks;
          if (reservation_fits(base, chunks, cap)) {
            const std::vector<int> p = park(rows[c], e, n, n);
            for (int j = 0; j < chunks; ++j) {
              if (items[base + j].cache != -1) fail("reservations overlap", e, n);
              items[base + j] = Item{c, j, base};
            }
            cache_parked[c] = p;
            handed[c] = true;
          } else {
            for (int i = 0; i < chunks; ++i) {
              const long it = (long)base + i;
              if (it >= 0 && it < cap) {
                if (items[it].cache != -1) fail("an empty mark overwrites an item", e, n);
                items[it].cache = -2;
              }
            }
          }
        }
        // in-place compactions (and the steps that move 128 rows or fewer)
        for (int c = 0; c < caches; ++c) {
          const int e = es[c], n = budget;
          if (handed[c] || e < 0 || e >= n) continue;
          for (int i = e; i < n; ++i) rows[c][i] = rows[c][i + 1];
          rows[c][n - 1] = n;
        }
        // the move kernel: items [0, queued) in a random order
        const int queued = items_queued(count, cap);
        std::vector<int> its(queued);
        for (int i = 0; i < queued; ++i) its[i] = i;
        std::shuffle(its.begin(), its.end(), rng);
        // reads of every chunk first, then the writes: the harshest interleaving
        std::vector<Chunk> cs(queued);
        for (int i : its) {
          const Item &it = items[i];
          if (it.cache == -1) fail("the move kernel reads an item no step wrote", i, queued);
          if (it.cache == -2) continue;
          const int e = es[it.cache], n = budget;
          chunk_read(rows[it.cache], cache_parked[it.cache], e, n, it.j, move_chunks(e, n), cs[i]);
        }
        for (int i : its) {
          const Item &it = items[i];
          if (it.cache < 0) continue;
          const int e = es[it.cache], n = budget;
          chunk_write(rows[it.cache], cache_parked[it.cache], e, n, it.j, move_chunks(e, n),
                      cs[i]);
        }
        for (int c = 0; c < caches; ++c) {
          const int e = es[c], n = budget;
          if (e < 0 || e == n) {                       // nothing evicted, or the incoming row
            for (int i = 0; i < n; ++i)
              if (rows[c][i] != i) fail("an untouched cache changed", e, n);
          } else {
            check_shifted(rows[c], e, n, n);
          }
        }
        ++launches;
      }
    }
  }
  return launches;
}

// Part 3: the pool header across a long sequence of calls.  Calls that hand
// nothing over launch no move kernel and leave the header alone.  In a call
// that does, every step workgroup records the phase it read and some reserve;
// the move kernel's workgroup 0 prepares the next call at a random moment
// among the other workgroups' reads.  Checked: every call starts on a zero
// counter, and every move workgroup reads exactly this call's reservations.
static long part3(std::mt19937 &rng) {
  int h[64] = {0};                                // the 256-byte header, zeroed before use
  // the launch phase, written with ordinary stores, shares no 128-byte line
  // with the words that atomics update
  if (kPoolLaunchPhase * 4 < 128 || kPoolLaunchPhase * 4 >= 256 || kPoolPhase * 4 >= 128 ||
      pool_counter(0) * 4 >= 128 || pool_counter(1) * 4 >= 128)
    fail("header layout", kPoolLaunchPhase, kPoolPhase);
  long calls = 0;
  for (int call = 0; call < 50000; ++call) {
    if (rng() % 4 == 0) continue;                 // nothing handed over
    const int p = h[kPoolPhase];
    if (h[pool_counter(p)] != 0) fail("a call starts on a counter that is not zero", p, call);
    const int wgs = 1 + (int)(rng() % 64);
    int reserved = 0;
    for (int b = 0; b < wgs; ++b) {
      h[kPoolLaunchPhase] = h[kPoolPhase];
      if (rng() % 3 == 0) {
        const int c = 2 + (int)(rng() % 190);
        h[pool_counter(h[kPoolPhase])] += c;
        reserved += c;
      }
    }
    const int grid = 1 + (int)(rng() % 1024);
    const int wg0_at = (int)(rng() % grid);
    for (int g = 0; g < grid; ++g) {
      if (g == wg0_at) {                          // workgroup 0's update
        const int mp = h[kPoolLaunchPhase];
        h[pool_counter(pool_next_phase(mp))] = 0;
        h[kPoolPhase] = pool_next_phase(mp);
      }
      const int lp = h[kPoolLaunchPhase];
      if (lp != p || h[pool_counter(lp)] != reserved)
        fail("a move workgroup reads another call's count", lp, call);
    }
    ++calls;
  }
  return calls;
}

int main() {
  std::mt19937 rng(20241202u);
  const long moves = part1(rng);
  const long launches = part2(rng);
  const long calls = part3(rng);
  std::printf("ok: %ld handed-over moves, %ld pooled launches, %ld calls through one header "
              "(chunk %d rows, handed over past %d rows)\n", moves, launches, calls, kMoveChunk,
              kDeferRows);
  return 0;
}
