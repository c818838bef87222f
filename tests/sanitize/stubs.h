// Interface of the launch stubs used by the host sanitizer harness.
#pragma once
#include <cstdint>

namespace stub {
void reset();                                 // forget the declared buffers
void declare(const void* p, uint64_t bytes);  // a buffer the next call may touch
long launches();                              // launches so far
long violations();                            // launches that touched undeclared memory
uint64_t addr(const void* p);
}  // namespace stub
