// Device error flags, one word per (device, stream).
//
// Kernels that see a non-finite input OR bit 0 into the flag word of the
// stream they run on; scmp_error_flags(stream) reads and clears that word
// only, so work on one stream never raises or clears another stream's flag.
// The words live in a fixed device array (no allocation); a stream gets its
// word the first time a flag-raising call runs on it.

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "internal.h"

namespace scmp {

constexpr int FLAG_SLOTS = 1024;
__device__ int g_stream_flags[FLAG_SLOTS];

namespace {

struct FlagRegistry {
  std::mutex mu;
  std::map<std::pair<int, hipStream_t>, int> slot;  // (device, stream) -> word
  std::map<int, int> used;                          // device -> words handed out
  std::map<int, int*> base;                         // device -> address of g_stream_flags
};

FlagRegistry& registry() {
  static FlagRegistry r;
  return r;
}

// Word of (device, stream), or -1 when the stream has none yet and `create`
// is false.  Caller holds the mutex.
int find_slot(FlagRegistry& r, int dev, hipStream_t st, bool create) {
  auto it = r.slot.find({dev, st});
  if (it != r.slot.end()) return it->second;
  if (!create) return -1;
  int& n = r.used[dev];
  if (n >= FLAG_SLOTS) return -2;
  r.slot[{dev, st}] = n;
  return n++;
}

int device_base(FlagRegistry& r, int dev, int** out) {
  auto it = r.base.find(dev);
  if (it == r.base.end()) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_stream_flags));
    if (e != hipSuccess || !p)
      return set_error(SCMP_ERR_HIP, std::string("flag words: ") + hipGetErrorString(e));
    it = r.base.emplace(dev, (int*)p).first;
  }
  *out = it->second;
  return SCMP_OK;
}

}  // namespace

int stream_flag(void* stream, int** out) {
  hipStream_t st = (hipStream_t)stream;
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  FlagRegistry& r = registry();
  std::lock_guard<std::mutex> lock(r.mu);
  int* base = nullptr;
  int s = device_base(r, dev, &base);
  if (s != SCMP_OK) return s;
  const int slot = find_slot(r, dev, st, true);
  if (slot < 0) return set_error(SCMP_ERR_ARG, "more than 1024 distinct streams raised flags on this device");
  *out = base + slot;
  return SCMP_OK;
}

int read_clear_stream_flags(void* stream, int* flags) {
  hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  int* word = nullptr;
  {
    FlagRegistry& r = registry();
    std::lock_guard<std::mutex> lock(r.mu);
    const int slot = find_slot(r, dev, st, false);
    if (slot >= 0) {
      int* base = nullptr;
      int s = device_base(r, dev, &base);
      if (s != SCMP_OK) return s;
      word = base + slot;
    }
  }
  // The stream is synchronised either way (the call's documented effect).
  int v = 0, zero = 0;
  if (word) e = hipMemcpyAsync(&v, word, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && v != 0) {
    e = hipMemcpyAsync(word, &zero, sizeof(int), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("flag readback: ") + hipGetErrorString(e));
  *flags |= v;
  return SCMP_OK;
}

}  // namespace scmp
