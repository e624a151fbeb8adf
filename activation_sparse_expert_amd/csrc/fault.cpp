// Allocation fault injection (host only): tests arm it to make the n-th
// allocation the library attempts fail, and check that every entry point then
// returns MOE_SEL_ENOMEM and leaves nothing allocated.
#include <atomic>

#include "internal.h"

namespace moe_sel {
namespace {
std::atomic<int> g_fault_countdown{0};  // 0: disarmed
}  // namespace

void arm_alloc_fault(int n) { g_fault_countdown.store(n > 0 ? n : 0); }

bool alloc_fault_hit() {
  int c = g_fault_countdown.load();
  while (c > 0) {
    if (g_fault_countdown.compare_exchange_weak(c, c - 1)) return c == 1;
  }
  return false;
}

}  // namespace moe_sel
