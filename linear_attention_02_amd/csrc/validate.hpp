// validate.hpp -- argument checks and launch planning for liblinattn, in plain
// C++ with no HIP dependency, so the host logic can be built and tested
// without a GPU (and under host sanitizers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/linattn.h"

namespace linattn {

struct Buffer {
  const void *ptr;
  size_t bytes;
  const char *name;
};

// Result of a check: status plus message for linattn_last_error().
struct Check {
  linattn_status status = LINATTN_OK;
  std::string message;
  bool ok() const { return status == LINATTN_OK; }
};

size_t dtype_bytes(linattn_dtype dt);  // 0 for an unknown type

// Launch plan for one forward call.
struct Plan {
  long long heads = 0;      // B * H
  long long chunks = 0;     // ceil(N / 64)
  int segments = 1;         // sequence segments per head (scan units)
  int seg_chunks = 0;       // chunks per segment
  int records = 0;          // state records per head in the workspace
  int ranges = 0;           // non-causal read ranges per head
  int range_chunks = 0;     // chunks per read range
  size_t workspace_bytes = 0;
};

// Plans a forward call.  `cus` is the device's compute-unit count, `override`
// a forced segment count (0 = automatic).
Plan plan_forward(long long heads, long long N, int causal, int cus, int override_segments);

Check check_forward(const void *Q, const void *K, const void *V, const void *O, int B, int H, int N, int C, int M,
                    linattn_dtype dt, const void *workspace, size_t workspace_bytes, size_t workspace_needed);

Check check_state_args(const float *S0, const float *z0, const float *S_out, const float *z_out, int B, int H,
                       const void *Q, const void *K, const void *V, const void *O, size_t qk_bytes,
                       size_t vo_bytes, const void *workspace, size_t workspace_bytes);

Check check_decode(const float *S, const float *z, const void *q, const void *k, const void *v, const float *o,
                   int BH, int C, int M, linattn_dtype dt);

bool overlaps(const Buffer &a, const Buffer &b);

}  // namespace linattn
