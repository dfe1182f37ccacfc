// kve_move_plan.h -- the geometry of a compaction handed from a step to the
// move kernel: which rows each chunk reads and writes, and which rows the
// step parks first.  Plain C++ (no HIP headers), so that the kernels and a
// host-side emulation of the protocol use the same code.
//
// A step that evicts stored row e of the n rows it held moves rows
// e+1 .. n-1 down one slot (keyformer_update step 3: later rows shift down,
// keeping temporal order) and puts the incoming row at n-1.  Handed over,
// the move is cut into chunks of kMoveChunk destination rows: chunk j fills
// destinations e + j*C .. min(e + (j+1)*C, n-1) - 1 from the row one above
// each.  The one source row that lies in the next chunk's destination range
// (its first destination) is read from a parked copy taken by the step before
// anything moved, and the incoming row waits in parked slot 0 until the last
// chunk writes it.  Every chunk therefore reads only rows that no other chunk
// writes, and the chunks may run in any order or at once.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define KVE_HD __host__ __device__
#else
#define KVE_HD
#endif

namespace kve {

// Rows per chunk of a handed-over compaction (one move-kernel workgroup
// each), and the longest move a step still does itself.  (Tuning builds may
// override the second with -D.)
constexpr int kMoveChunk = 64;
#ifndef KVE_DEFER_ROWS
#define KVE_DEFER_ROWS (2 * kMoveChunk)
#endif
constexpr int kDeferRows = KVE_DEFER_ROWS;

// Whether a step that held n rows and evicted row e (-1: none; n: the
// incoming row) hands its move over: only moves of more than kDeferRows rows.
KVE_HD inline bool move_handed_over(int e, int n) {
  return e >= 0 && e < n - 1 && n - 1 - e > kDeferRows;
}

// Chunks of the move of rows e+1 .. n-1 (n - 1 - e rows).
KVE_HD inline int move_chunks(int e, int n) { return (n - 1 - e + kMoveChunk - 1) / kMoveChunk; }

// Chunks of the longest move a cache of at most `budget` stored rows can
// make (row 0 evicted: budget - 1 rows move); at least 1.
KVE_HD inline int max_move_chunks(int budget) {
  const int c = (budget - 1 + kMoveChunk - 1) / kMoveChunk;
  return c > 1 ? c : 1;
}

// First destination row of chunk j, and the last destination of the move.
KVE_HD inline int chunk_first_dst(int e, int j) { return e + j * kMoveChunk; }
KVE_HD inline int move_last_dst(int n) { return n - 2; }

// The cache row parked in slot j >= 1 before anything moves: chunk j's first
// destination, which chunk j-1 reads as its last source.  (Slot 0 holds the
// incoming row.)
KVE_HD inline int parked_row(int e, int j) { return chunk_first_dst(e, j); }

// Where chunk j (of `chunks`) reads the source of destination `dst`: the
// cache row dst + 1, or (return -1) parked slot j + 1 when that row is the
// next chunk's first destination.
KVE_HD inline int chunk_source_row(int e, int j, int chunks, int dst) {
  const int src = dst + 1;
  if (j + 1 < chunks && src == chunk_first_dst(e, j + 1)) return -1;
  return src;
}

// Whether a reservation of `chunks` items starting at `base` (the value the
// pool counter held before the reserving atomic added them) lies inside a
// pool of `cap` items.  One that does not is marked empty where it overlaps
// the pool, and its cache compacts in place.
KVE_HD inline bool reservation_fits(int base, int chunks, int cap) {
  return base >= 0 && chunks >= 1 && base <= cap - chunks;
}

// Items the move kernel reads: every reservation counted, but none past the
// pool's end.
KVE_HD inline int items_queued(int reserved, int cap) { return reserved < cap ? reserved : cap; }

// The pool's header: 32-bit words that the calls keep consistent among
// themselves (all zero before the first call):
//   kPoolCount + 0, + 1   reservation counters of even and odd phases
//   kPoolPhase            phase of the next call
//   kPoolLaunchPhase      phase the last step launch used (on a cache line of
//                         its own, written with ordinary stores, apart from
//                         the words that atomics update)
// A step launch reads the phase p, reserves on counter pool_counter(p) --
// zero at that point -- and records p for the move kernel.  The move kernel
// reads p and counter pool_counter(p); its workgroup 0 zeroes the other
// counter, which no one reads until the next call, and sets the phase to
// p + 1.  So no counter is contended by the move kernel's workgroups, and
// each call starts with its counter at zero without any clearing by the host.
constexpr int kPoolCount = 0;
constexpr int kPoolPhase = 2;
constexpr int kPoolLaunchPhase = 32;          // byte 128 of the 256-byte header
KVE_HD inline int pool_counter(int phase) { return kPoolCount + (phase & 1); }
KVE_HD inline int pool_next_phase(int phase) { return (phase + 1) & 0x3fffffff; }

}  // namespace kve
