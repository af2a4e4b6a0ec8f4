// Stand-in marker library for the CPU test of the runtime's trace ranges: prints every
// range push and pop with its nesting depth instead of handing it to a profiler.
#include <cstdio>

static int depth = 0;

extern "C" int roctxRangePushA(const char* message) {
  std::printf("roctx push %d %s\n", depth, message);
  return depth++;
}

extern "C" int roctxRangePop() {
  --depth;
  std::printf("roctx pop %d\n", depth);
  return depth;
}
