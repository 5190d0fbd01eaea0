// What the host-only launcher stand-ins saw (sanitized build of the validation layer).
#pragma once
#include <cstdint>

namespace stub {
struct Record {
  int lossless = 0, bias32 = 0, exact = 0, merge = 0, patch = 0, bwd = 0;
  int last_phase = -1, last_tile = -1;
  uintptr_t ws_lo = 0, ws_hi = 0;  // the caller's workspace [lo, hi) of the current call
};
extern Record rec;
void expect_inside(const void* p, size_t bytes, const char* what);
}  // namespace stub
