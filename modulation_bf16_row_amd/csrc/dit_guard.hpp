// dit_guard.hpp -- host-side argument checks shared by the C entry points
// (dit_abi.cpp, and the probe entry points of the instrumented build).
// Pure host code; nothing here touches a GPU.
#pragma once

#include <stdint.h>

#include "dit.h"

namespace dit {
namespace guard {

// Largest byte extent a tensor argument may describe, from its first
// element to one past its last: 2^56 bytes (64 PiB), beyond any device
// memory, and small enough that every offset the kernels form from it fits
// an int64_t with room to spare.
constexpr int64_t kMaxExtentBytes = int64_t(1) << 56;

// Records the reason for the calling thread and returns s.
dit_status_t fail(dit_status_t s, const char *why);

// The calling thread's most recent reason ("" if none).
const char *reason();

dit_status_t hip_status(hipError_t e);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True when a strided set of `count` segments of `len` elements, `step`
// elements apart, starting at p (elements of `esz` bytes) spans at most
// kMaxExtentBytes and does not run past the end of the address space.
// Arguments must be non-negative; the arithmetic cannot overflow.
bool extent_ok(const void *p, int64_t step, int64_t count, int64_t len, int64_t esz);

// A set of byte segments [base + i*step, base + i*step + len), i < count.
struct Span {
  uintptr_t base;
  int64_t step;
  int64_t count;
  int64_t len;
};

// True if some byte belongs to both spans.  Exact when both have the same
// step (or one has a single segment); otherwise compares the hulls, which
// may report an overlap that the segments avoid (the safe direction).
// Computed in 128-bit integers, so any non-negative int64_t fields are safe.
bool spans_overlap(Span a, Span b);

}  // namespace guard
}  // namespace dit
