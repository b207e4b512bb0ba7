// Launch timing: RAII bracket recording HIP events around one kernel launch.
#pragma once

#include "common.h"

namespace egnn {

bool timing_on();
void timing_begin(hipStream_t s, int *slot);
void timing_end(hipStream_t s, int slot, const char *name, double flops, double bytes);

struct Timed {
  hipStream_t s;
  const char *name;
  double flops, bytes;
  int slot = -1;
  Timed(hipStream_t st, const char *n, double f, double b) : s(st), name(n), flops(f), bytes(b) {
    if (timing_on()) timing_begin(s, &slot);
  }
  ~Timed() {
    if (slot >= 0) timing_end(s, slot, name, flops, bytes);
  }
};

}  // namespace egnn
