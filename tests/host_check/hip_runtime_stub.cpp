// Stand-in definitions of the HIP runtime entry points that the library's host code and the
// compiler-generated kernel stubs call (module registration, launch configuration, launch, function
// attributes, error query, device queries). Each launch is checked against HIP's launch limits and the gfx950
// LDS budget; a violation prints what it saw and aborts the process.
#include "hip_runtime_stub.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>

namespace {

struct Config {
  dim3 grid, block;
  size_t lds;
  hipStream_t stream;
};

// State lives in function-local statics: the module constructors that register kernels run before
// this file's namespace-scope objects would be constructed.
struct State {
  std::vector<StubLaunch> launches;
  long calls = 0;
  std::map<const void*, std::string> names;     // host stub -> device symbol
  std::map<const void*, int> max_dynamic_lds;   // opt-in above the default 64 KiB
  std::vector<Config> config_stack;
};

State& state() {
  static State s;
  return s;
}

constexpr size_t kDefaultDynamicLds = 64 * 1024;
constexpr size_t kLdsPerWorkgroup = 160 * 1024;   // gfx950

[[noreturn]] void fail(const char* what, const std::string& kernel, dim3 g, dim3 b, size_t lds) {
  std::fprintf(stderr,
               "HIP stub: %s (kernel %s, grid %u x %u x %u, block %u x %u x %u, dynamic LDS %zu)\n",
               what, kernel.c_str(), g.x, g.y, g.z, b.x, b.y, b.z, lds);
  std::abort();
}

}  // namespace

std::vector<StubLaunch>& stub_launches() { return state().launches; }
long stub_hip_calls() { return state().calls; }
void stub_clear() {
  state().launches.clear();
  state().calls = 0;
}

extern "C" {

// Module registration, emitted by the compiler into every translation unit that holds kernels.
void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}

void __hipRegisterFunction(void**, const void* host_function, char*, const char* device_name, int,
                           void*, void*, void*, void*, int*) {
  state().names[host_function] = device_name ? device_name : "?";
}

void __hipUnregisterFatBinary(void**) {}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
  state().config_stack.push_back(Config{grid, block, lds, stream});
  return hipSuccess;
}

hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* lds, hipStream_t* stream) {
  if (state().config_stack.empty()) {
    std::fprintf(stderr, "HIP stub: launch configuration popped without a push\n");
    std::abort();
  }
  const Config c = state().config_stack.back();
  state().config_stack.pop_back();
  *grid = c.grid;
  *block = c.block;
  *lds = c.lds;
  *stream = c.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void* function, dim3 grid, dim3 block, void** args, size_t lds,
                           hipStream_t) {
  ++state().calls;
  const auto it = state().names.find(function);
  const std::string name = it == state().names.end() ? "<unregistered>" : it->second;
  if (it == state().names.end()) fail("launch of an unregistered function", name, grid, block, lds);
  if (!args) fail("launch without an argument array", name, grid, block, lds);
  const uint64_t threads = (uint64_t)block.x * block.y * block.z;
  if (threads == 0 || threads > 1024) fail("block size outside [1, 1024]", name, grid, block, lds);
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) fail("empty grid", name, grid, block, lds);
  // the dispatch packet carries the grid in work-items, 32 bits per dimension
  if ((uint64_t)grid.x * block.x >= ((uint64_t)1 << 32) ||
      (uint64_t)grid.y * block.y >= ((uint64_t)1 << 32) ||
      (uint64_t)grid.z * block.z >= ((uint64_t)1 << 32))
    fail("2^32 or more work-items along a grid dimension", name, grid, block, lds);
  if (lds > kLdsPerWorkgroup) fail("dynamic LDS above 160 KiB", name, grid, block, lds);
  if (lds > kDefaultDynamicLds) {
    const auto opt = state().max_dynamic_lds.find(function);
    if (opt == state().max_dynamic_lds.end() || (size_t)opt->second < lds)
      fail("dynamic LDS above 64 KiB without a matching opt-in", name, grid, block, lds);
  }
  state().launches.push_back(StubLaunch{name, grid, block, lds});
  return hipSuccess;
}

hipError_t hipFuncSetAttribute(const void* function, hipFuncAttribute attr, int value) {
  ++state().calls;
  if (attr == hipFuncAttributeMaxDynamicSharedMemorySize) {
    if (value < 0 || (size_t)value > kLdsPerWorkgroup) {
      std::fprintf(stderr, "HIP stub: dynamic LDS opt-in of %d bytes\n", value);
      std::abort();
    }
    state().max_dynamic_lds[function] = value;
  }
  return hipSuccess;
}

hipError_t hipGetLastError(void) {
  ++state().calls;
  return hipSuccess;
}

// Device queries: one MI355X (256 CUs) as device 0.
hipError_t hipGetDevice(int* device) {
  ++state().calls;
  if (!device) return hipErrorInvalidValue;
  *device = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  ++state().calls;
  if (!value || device != 0) return hipErrorInvalidValue;
  *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}

}  // extern "C"
