// Host-side pipeline planner: stage/order validation, buffer version counts
// and LDS arena packing.  Plain C++, no HIP.
//
//  * Validation follows TileLang ch.22 ("pipeline-sync-multibuffer") §2.2:
//    no two statements share an order, and a statement that reads a buffer
//    another one writes may not sit in an earlier stage than the writer, nor
//    (same stage) come before it in order.
//  * Versions follow §2.4: a buffer first written in stage `def` and last
//    read in stage `use` needs use - def + 1 versions; a buffer the pipeline
//    never writes keeps one; when the count is at least two it drops by one
//    unless some writer precedes some reader both in order and in stage
//    (every access of a buffer is taken to overlap every other).
//  * Packing follows §3.3: each buffer (all its versions, one block) is live
//    over an interval of program points; blocks are placed in order of
//    (start, larger first, index); blocks whose interval has ended go back
//    to a free list that is kept sorted and coalesced; a block takes the
//    free hole that wastes least after alignment, else new space at the top
//    of the arena.  A free hole that reaches the top of the arena counts as
//    part of that top space (the block starts at the hole, aligned, and the
//    arena grows by the rest).
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

namespace pgemm {
namespace planner {

struct Access {
  int stmt, buffer;
  bool write;
};

// Returns false if the (stage, order) annotation is invalid.
inline bool validate(const std::vector<int> &stage, const std::vector<int> &order, const std::vector<Access> &acc) {
  const size_t n = stage.size();
  if (order.size() != n) return false;
  for (size_t i = 0; i < n; ++i)
    for (size_t j = i + 1; j < n; ++j)
      if (order[i] == order[j]) return false;
  for (const Access &w : acc) {
    if (!w.write) continue;
    for (const Access &r : acc) {
      if (r.write || r.buffer != w.buffer || r.stmt == w.stmt) continue;
      const int sw = stage[w.stmt], sr = stage[r.stmt];
      if (sw > sr) return false;
      if (sw == sr && order[w.stmt] > order[r.stmt]) return false;
    }
  }
  return true;
}

// Stage and order of every statement that writes, and of every statement
// that reads, one buffer.
struct BufferUses {
  struct Point {
    int stage, order;
  };
  std::vector<Point> writes, reads;
};

inline BufferUses uses_of(int buffer, const std::vector<int> &stage, const std::vector<int> &order,
                          const std::vector<Access> &acc) {
  BufferUses u;
  for (const Access &a : acc)
    if (a.buffer == buffer) (a.write ? u.writes : u.reads).push_back({stage[a.stmt], order[a.stmt]});
  return u;
}

// Copies of `buffer` the pipelined loop keeps.  A value written in stage d
// and last read in stage u is alive across u - d iteration boundaries, so
// u - d + 1 copies (the ring's slots); a buffer the loop never writes needs
// its one copy.  One copy fewer suffices when no write reaches a read that
// comes later in the body and in a later stage: then every read of an
// iteration's value happens before the body writes the next one.
inline int versions(int buffer, const std::vector<int> &stage, const std::vector<int> &order,
                    const std::vector<Access> &acc) {
  const BufferUses u = uses_of(buffer, stage, order, acc);
  if (u.writes.empty()) return 1;
  auto by_stage = [](const BufferUses::Point &x, const BufferUses::Point &y) { return x.stage < y.stage; };
  const int first_write = std::min_element(u.writes.begin(), u.writes.end(), by_stage)->stage;
  int last_read = first_write;  // a buffer written but not read later lives within its stage
  if (!u.reads.empty()) last_read = std::max(last_read, std::max_element(u.reads.begin(), u.reads.end(), by_stage)->stage);
  const int span = last_read - first_write + 1;
  const bool carried = std::any_of(u.writes.begin(), u.writes.end(), [&](const BufferUses::Point &w) {
    return std::any_of(u.reads.begin(), u.reads.end(), [&](const BufferUses::Point &r) {
      return w.order < r.order && w.stage < r.stage;
    });
  });
  return span >= 2 && !carried ? span - 1 : span;
}

struct Block {
  int64_t bytes;  // all versions
  int64_t align;  // power of two
  int start, end; // live over [start, end)
};

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Hole {
  int64_t lo, hi;
};

// Returns [lo, hi) to a free list kept sorted by address and coalesced.
inline void free_range(std::vector<Hole> *list, int64_t lo, int64_t hi) {
  if (hi <= lo) return;
  auto it = std::lower_bound(list->begin(), list->end(), lo, [](const Hole &x, int64_t v) { return x.lo < v; });
  size_t k = (size_t)(it - list->begin());
  list->insert(it, Hole{lo, hi});
  if (k + 1 < list->size() && (*list)[k].hi == (*list)[k + 1].lo) {
    (*list)[k].hi = (*list)[k + 1].hi;
    list->erase(list->begin() + (long)k + 1);
  }
  if (k > 0 && (*list)[k - 1].hi == (*list)[k].lo) {
    (*list)[k - 1].hi = (*list)[k].hi;
    list->erase(list->begin() + (long)k);
  }
}

// Places the blocks; fills offsets and returns the arena size.
inline int64_t pack(const std::vector<Block> &blocks, std::vector<int64_t> *offsets) {
  const size_t n = blocks.size();
  offsets->assign(n, 0);
  std::vector<size_t> idx(n);
  for (size_t i = 0; i < n; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) {
    if (blocks[a].start != blocks[b].start) return blocks[a].start < blocks[b].start;
    if (blocks[a].bytes != blocks[b].bytes) return blocks[a].bytes > blocks[b].bytes;
    return a < b;
  });
  std::vector<Hole> holes;
  std::vector<size_t> live;
  int64_t top = 0;
  for (size_t i : idx) {
    const Block &b = blocks[i];
    std::vector<size_t> still;  // intervals ended by this start return their space
    for (size_t j : live) {
      if (blocks[j].end <= b.start)
        free_range(&holes, (*offsets)[j], (*offsets)[j] + blocks[j].bytes);
      else
        still.push_back(j);
    }
    live.swap(still);
    long best = -1;
    int64_t best_waste = 0;
    for (size_t h = 0; h < holes.size(); ++h) {
      const int64_t at = align_up(holes[h].lo, b.align);
      if (at + b.bytes > holes[h].hi) continue;
      const int64_t waste = (holes[h].hi - holes[h].lo) - b.bytes;
      if (best < 0 || waste < best_waste) {
        best = (long)h;
        best_waste = waste;
      }
    }
    int64_t off;
    if (best >= 0) {
      const Hole h = holes[(size_t)best];
      holes.erase(holes.begin() + best);
      off = align_up(h.lo, b.align);
      free_range(&holes, h.lo, off);
      free_range(&holes, off + b.bytes, h.hi);
    } else {
      int64_t from = top;
      if (!holes.empty() && holes.back().hi == top) {  // the top hole grows
        from = holes.back().lo;
        holes.pop_back();
      }
      off = align_up(from, b.align);
      free_range(&holes, from, off);
      top = off + b.bytes;
    }
    (*offsets)[i] = off;
    live.push_back(i);
  }
  return top;
}

}  // namespace planner
}  // namespace pgemm
