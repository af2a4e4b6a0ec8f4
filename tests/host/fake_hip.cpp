// A stand-in for the few HIP runtime calls the host runtime (runtime.cpp) makes, for a
// CPU test program: pinned buffers are plain host memory, events and streams do
// nothing, and every host-to-device copy (the per-call metadata uploads, which carry
// the page-table updates) is recorded in g_uploads instead of being performed, so a
// test can compare what two contexts would have sent to the device. Device addresses
// are never dereferenced.
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

std::vector<std::vector<unsigned char>> g_uploads;

namespace {
struct FakeEvent {
  int tag;
};
}  // namespace

hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int) {
  *ptr = std::malloc(size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = (hipEvent_t) new FakeEvent{1};
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete (FakeEvent*)e;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.f;
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void*, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t) {
  if (kind == hipMemcpyHostToDevice) {
    const unsigned char* p = (const unsigned char*)src;
    g_uploads.emplace_back(p, p + bytes);
  }
  return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stand-in HIP runtime"; }
