// Host AdamW of the offload path (internal).
#pragma once

#include <stdint.h>

namespace zs {

// The step's fp32 scalars plus the gradient factor k (1, or a clip coefficient).
struct HostScalars {
  float b1, c1, b2, c2, e, ss, rb, dk, k;
};

// P, M, V updated in place from g*k; B = bf16(P).  All host memory.
// Runs on up to `threads` threads (ranges no thread could be started for run on
// the caller's thread); throws only std::bad_alloc, before touching any element.
void cpu_adam(const float* g, int64_t n, float* P, float* M, float* V, uint16_t* B, const HostScalars& c,
              int threads);

}  // namespace zs
