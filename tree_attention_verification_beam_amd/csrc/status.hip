// status.hip -- the library's own device status word and the host call that
// reads a status word after the work that wrote it.
//
// Faults that only the device can see (a bad parent index, a token outside the
// vocabulary, a context past the cache) are OR-ed into an int32 status word by
// the kernels, since the calls return before their kernels run.  A caller may
// pass its own word to every call; a call that gets none uses the library's
// word on the current device, a file-scope device variable whose address is
// looked up once per device.
#include <mutex>

#include "common.hpp"

namespace spec {
namespace {

__device__ int32_t g_status_word;  // one per device, zero at load

constexpr int kMaxDevices = 64;

std::mutex g_status_mu;
int32_t* g_status_ptr[kMaxDevices];  // per-device address of g_status_word

// Address of the library's status word on the current device (nullptr if the
// runtime cannot give it).
int32_t* library_status_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_status_mu);
  if (!g_status_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_status_word)) != hipSuccess) return nullptr;
    g_status_ptr[dev] = static_cast<int32_t*>(p);
  }
  return g_status_ptr[dev];
}

}  // namespace

int32_t* status_or_library(int32_t* status) {
  return status ? status : library_status_word();
}

}  // namespace spec

using namespace spec;

extern "C" int spec_last_device_status(const int32_t* status_dev, void* stream) {
  int32_t* word = status_dev ? const_cast<int32_t*>(status_dev) : library_status_word();
  if (!word) return SPEC_ERR_HIP;
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return SPEC_ERR_HIP;
  int32_t v = 0;
  if (hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return SPEC_ERR_HIP;
  if (!status_dev) {
    // the library's own word is cleared once read (a caller's word never is)
    const int32_t zero = 0;
    if (hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
      return SPEC_ERR_HIP;
  }
  return v & 0x7fffffff;
}
