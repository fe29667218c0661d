// schedule.cpp -- ring task list and chunk sizes (host side).
#include "schedule.hpp"

#include <math.h>

namespace hc {

size_t chunk_elems(size_t count, double fraction, size_t align) {
  if (align == 0 || !(fraction > 0.0) || fraction > 1.0) return 0;
  double want = ceil((double)count * fraction);
  size_t c = round_up((size_t)want, align);
  return c == 0 ? align : c;
}

std::vector<hc_task_t> ring_tasks(int R, size_t count, size_t chunk) {
  std::vector<hc_task_t> out;
  if (R < 1 || chunk == 0) return out;
  const size_t L = ceil_div(count, (size_t)R);
  for (int phase = 0; phase < 2; ++phase) {
    for (int s = 0; s + 1 < R; ++s) {
      for (int q = 0; q < R; ++q) {
        const int j = ring_slice(phase, q, s, R);
        size_t lo = (size_t)j * L, hi = lo + L;
        if (lo > count) lo = count;
        if (hi > count) hi = count;
        const size_t nchunks = ceil_div(hi - lo, chunk);
        for (size_t c = 0; c < nchunks; ++c) {
          hc_task_t t;
          t.src = ring_mod(q - 1, R);
          t.dst = q;
          t.step = s;
          t.chunk = (int32_t)c;
          t.op = phase == 0 ? 1 : 2;
          t.slice = j;
          t.off = lo + c * chunk;
          t.len = (hi - t.off) < chunk ? (hi - t.off) : chunk;
          out.push_back(t);
        }
      }
    }
  }
  return out;
}

}  // namespace hc
