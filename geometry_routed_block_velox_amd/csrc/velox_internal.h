// Internal declarations shared by the HIP translation units of libvelox.
// Not part of the public ABI (include/velox.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "velox.h"
#include "velox_host.h"
#include "velox_launch.h"

namespace velox {

// Number of XCDs of an MI355X; workgroups are dispatched round-robin over them.
constexpr int kNumXcd = 8;

// Map a dispatch-order workgroup id to a work item so that consecutive work
// items run on the same XCD (and share its L2): XCD x receives the items
// [x*per, (x+1)*per).  Identity when the grid does not divide evenly.
__device__ __forceinline__ int xcd_grouped(int wg, int nwg) {
  if (nwg % kNumXcd) return wg;
  const int per = nwg / kNumXcd;
  return (wg % kNumXcd) * per + wg / kNumXcd;
}

}  // namespace velox
