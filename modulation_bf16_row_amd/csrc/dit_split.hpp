// dit_split.hpp -- the split-row layout of the row kernels (LayerNorm + AdaLN,
// the gated residual + LN producer, RMSNorm-scale), taken where the staged
// layout of dit_rows.hpp does not apply (per-token modulation, or too few rows
// per modulation row).
//
// Layout.  One workgroup per row at a time, W = ceil(NC / 2) waves; wave w
// moves chunks 2w and 2w + 1 of the row (1 KiB each per operand, the same
// lane-to-element map as the row layout: lane l holds elements 512c + 8l ..
// 512c + 8l + 7 of chunk c).  A wave that streams a whole 10 KiB row per
// operand keeps ten 1 KiB accesses per operand in flight; on MI355X a copy
// in that pattern runs 525-530 us at the Wan 720p LayerNorm shape (three
// 10 KiB row inputs, one output) against 490 us when each wave moves two
// chunks and 480 us when it moves one, independent of the order in which a
// wave walks its chunks.  Two chunks per wave balance the short bursts
// against the rows a CU keeps in flight (a row ties up W waves, and at most
// 32 waves are resident per CU): at that shape one chunk per wave ran the
// LayerNorm about 30% slower than two, three or five chunks 5-8% slower.
//
// The sum order is unchanged.  The reduction of a row needs, for each lane
// l, its terms in (chunk, element) order, a chain that runs through every
// chunk; so the waves publish their x chunks (bf16, 16 bytes per lane and
// chunk) to LDS, wave 0 runs the chains of order R over the published row
// and the fixed butterfly, and leaves the row's statistics in LDS for all
// waves.  Each wave keeps its own chunks in registers for the output.  The
// register budget is 8 waves per SIMD (64 VGPRs): a split kernel left at the
// compiler's own choice of 84 VGPRs holds fewer rows per CU and ran 25%
// slower than the same code at 64.
//
// Every load is issued with its index clamped into the tensor (chunks past
// the row reload element 0, whose values are never used), so the loads carry
// no branches.
#pragma once

#include "dit_rows.hpp"

namespace dit {

constexpr int kSplitChunks = 2;                       // chunks per wave

template <int NC>
constexpr int split_waves() {
  return (NC + kSplitChunks - 1) / kSplitChunks;
}

// Largest workgroup: NC = 16, eight waves.
constexpr int kSplitMaxThreads = 64 * split_waves<16>();

#define DIT_SPLIT_KERNEL DIT_SPLIT_KERNEL_W(8)
// A smaller budget for kernels that do not fit 64 VGPRs (W waves per SIMD).
#define DIT_SPLIT_KERNEL_W(W) \
  __launch_bounds__(kSplitMaxThreads) __attribute__((amdgpu_waves_per_eu(W, 8)))

// Chunk k of wave w.
__device__ __forceinline__ int split_chunk(int w, int k) { return w * kSplitChunks + k; }

// Chunk c exists and this lane's vector of it lies inside the row?
template <int NC>
__device__ __forceinline__ bool split_has(int c, int lane, int dim) {
  return c < NC && valid<NC>(c, lane, dim);
}

// Element offset of this lane's vector of chunk c, clamped to 0 outside the row.
template <int NC>
__device__ __forceinline__ int split_col(int c, int lane, int dim) {
  return split_has<NC>(c, lane, dim) ? 512 * c + 8 * lane : 0;
}

// This wave's chunks of one row; STREAM selects the nontemporal policy.
template <int NC, bool STREAM>
__device__ __forceinline__ void split_load(V8 (&v)[kSplitChunks], const uint16_t *row, int w,
                                           int lane, int dim) {
#pragma unroll
  for (int k = 0; k < kSplitChunks; ++k) {
    const uint16_t *p = row + split_col<NC>(split_chunk(w, k), lane, dim);
    v[k] = STREAM ? load8_stream(p) : load8(p);
  }
}

// The published row: chunk c of lane l at xs[64c + l] (16 bytes, so a wave's
// 64 lanes touch 1 KiB of consecutive LDS: no bank conflicts).
template <int NC>
__device__ __forceinline__ void split_publish(uint4 *xs, const V8 (&v)[kSplitChunks], int w,
                                              int lane) {
#pragma unroll
  for (int k = 0; k < kSplitChunks; ++k) {
    const int c = split_chunk(w, k);
    if (c < NC) xs[64 * c + lane] = make_uint4(v[k].w[0], v[k].w[1], v[k].w[2], v[k].w[3]);
  }
}

__device__ __forceinline__ V8 split_fetch(const uint4 *xs, int c, int lane) {
  const uint4 u = xs[64 * c + lane];
  return V8{{u.x, u.y, u.z, u.w}};
}

// f(c, chunk c) for c = 0 .. NC - 1 in order, over the published row.  The
// LDS reads run one chunk ahead of f, and a scheduling barrier closes each
// step: without it the compiler issues the reads of the whole row at once,
// which takes 4 NC VGPRs and spills under the 64-VGPR budget from NC = 4.
template <int NC, class F>
__device__ __forceinline__ void split_walk(const uint4 *xs, int lane, F f) {
  constexpr int kAhead = 1;
  V8 buf[kAhead + 1];
#pragma unroll
  for (int c = 0; c < kAhead && c < NC; ++c) buf[c] = split_fetch(xs, c, lane);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c + kAhead < NC) buf[(c + kAhead) % (kAhead + 1)] = split_fetch(xs, c + kAhead, lane);
    f(c, buf[c % (kAhead + 1)]);
    phase_barrier();
  }
}

// Grid: one workgroup per row up to the grid limit; a workgroup then walks
// the rows gridDim.x apart.
inline dim3 split_grid(int64_t rows) {
  return dim3((unsigned)(rows < 0x7FFFFFFF ? rows : 0x7FFFFFFF));
}

}  // namespace dit
