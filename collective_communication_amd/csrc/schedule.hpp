// schedule.hpp -- ring schedule and chunking (host side).
//
// The ring follows the primitives of "ResCCL: Resource-Efficient Scheduling
// for Collective Communication" (section 1: send, recv, recvReduceCopy; a
// chunk is about 1% of the data) written as its Transfer(srcRank, dstRank,
// step, chunkId, opType) tasks (section 3).  Data dependencies exist only
// inside one chunk, across steps (section 3, dependency analysis), which is
// what lets a launcher group a whole step's chunks into one kernel.
//
// Ring indexing (the pages give none): reduce-scatter step s, receiver q
// gets slice (q-2-s) mod R from q-1; all-gather step s, receiver q gets slice
// (q-1-s) mod R from q-1.  After the reduce-scatter rank r owns slice r.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "hc.h"

namespace hc {

inline int ring_mod(int a, int r) { int m = a % r; return m < 0 ? m + r : m; }
inline size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return ceil_div(a, b) * b; }

// Slice owned by receiver q at a reduce-scatter (phase 0) or all-gather
// (phase 1) step.
inline int ring_slice(int phase, int q, int step, int R) {
  return phase == 0 ? ring_mod(q - 2 - step, R) : ring_mod(q - 1 - step, R);
}

// Chunk in elements: ceil(count * fraction) rounded up to align.
size_t chunk_elems(size_t count, double fraction, size_t align);

// The allreduce task list in execution order.
std::vector<hc_task_t> ring_tasks(int R, size_t count, size_t chunk);

}  // namespace hc
