// A stand-in for the HIP runtime's launch interface (hip_runtime_stub.cpp): with it the library's
// host code, the validation of the C entry points and the launchers' set-up, runs on a machine with
// no GPU, under AddressSanitizer and UndefinedBehaviorSanitizer. Launches are checked against
// HIP's limits and recorded, never run.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <string>
#include <vector>

struct StubLaunch {
  std::string kernel;   // device symbol name, as the module constructor registered it
  dim3 grid, block;
  size_t dynamic_lds;
};

// Launches recorded since the last clear, in order.
std::vector<StubLaunch>& stub_launches();
// HIP calls of any kind (launch, attribute, error query) since the last clear.
long stub_hip_calls();
void stub_clear();
