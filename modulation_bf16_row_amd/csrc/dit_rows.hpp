// dit_rows.hpp -- shared pieces of the gfx950 row kernels, whose rows carry a
// reduction (dit_ln.hip, dit_gate_ln.hip, dit_rms.hip): geometry, row and
// modulation loads, binary32 LDS staging, row runs and launch shapes.  The
// elementwise kernels (dit_gate.hip, dit_mod.hip) use the vector helpers and
// load policies only.
//
// Geometry.  One 64-lane wave per row at a time; lane l owns the 8-element
// vectors at 512c + 8l of chunk c (c < NC = ceil(dim / 512)), each moved
// with one 128-bit access, so a wave-wide access is 1 KiB contiguous.  A
// wave walks a contiguous run of `rows_per_wave` rows of its workgroup
// (four waves).  The row stays in VGPRs between the LayerNorm passes, so x
// is read from HBM once; latency is hidden by the other waves resident on
// the SIMD.  Outputs move with the nontemporal cache policy, row inputs
// with the per-kernel policy below, shared operands with the default one.
//
// Modulation operands.  With per-batch modulation the grid is laid out per
// modulation row: blocks_per_mod workgroups cover the rows of one
// modulation row, so all rows of a workgroup share it.  The workgroup
// converts its per-element operands once into LDS as binary32 values --
// bf(1 + scale) and shift, the RMSNorm weight and scale, tanh(gate), or
// gate, bf(1 + scale) and shift -- and the waves read them with two 128-bit LDS accesses per
// 8-element vector, with no bf16 unpacking in the row loop (the kernels
// are close to their vector-ALU budget, so every instruction per element
// counts).  Without the staged layout (per-token modulation) LayerNorm, the
// gated residual + LN producer and RMSNorm-scale split each row over several
// waves (dit_split.hpp); RMSNorm-tanh-residual lays its rows out
// consecutively, one per wave, and each wave loads its row's gate row.
//
// Sums follow R(dim): each lane adds its own terms in (chunk, element)
// order, then a fixed xor butterfly across the 64 lanes.
//
// Sources: AdaLN rounding points -- page "基于Agent的SGLang扩散模型Kernel优化实践"
// (tahou.com), section "数学等价不代表结果完全一致"; gated residual +
// LayerNorm/AdaLN producer -- same page, sections "将FP8量化融合到前序算子" and
// "NVFP4的三组优化"; native bf16 RMSNorm chain -- page "#34085 [diffusion] Clean
// up kernels and shared fast paths", section "关键源码片段";
// rmsnorm+tanh(gate)*x+residual -- page "AI Agent 驱动的 SGLang Kernel
// 一等公民", section 0x3 / 3.2.
#pragma once

#include "dit_device.hpp"
#include "dit_launch.hpp"

namespace dit {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;
static_assert(kThreads >= kTanhTabVecs, "one workgroup copies the tanh table in one pass");

// Load policy of the streamed row inputs, per kernel, as measured on MI355X
// (Qwen-Image and Wan shapes): the nontemporal policy helps the kernels that
// read two or more row streams and slows the single-stream norms.
// The gated residual + LN producer reads its residual nontemporal and y with
// the default policy (kNtGateLnY): 38.0 against 41.0 us at the Qwen-Image
// shape, in a DiT-order sequence with the QKV and RMSNorm epilogues after it,
// which it does not slow.  The same split in the standalone gate-add and
// tanh-residual made those faster back to back but slowed LN and RMS-scale in
// the five-kernel step by ~4 us each, so they keep both streams nontemporal.
constexpr bool kNtLn = false, kNtRms = false, kNtTanh = true, kNtGate = true, kNtMod = false;
constexpr bool kNtGateLnY = false;

// Register budget: at least W6 waves per SIMD at dim <= 3072 (NC <= 6),
// scaled down in proportion (rounded) for longer rows.
constexpr int waves_per_simd(int nc, int w6) {
  return nc <= 6 ? w6 : ((w6 * 6 + nc / 2) / nc > 1 ? (w6 * 6 + nc / 2) / nc : 1);
}
#define DIT_OCCUPANCY(NC, W6) __attribute__((amdgpu_waves_per_eu(waves_per_simd(NC, W6), 8)))

// Chunk c of this lane lies inside the row?  Chunks before the last are full.
template <int NC>
__device__ __forceinline__ bool valid(int c, int lane, int dim) {
  return c < NC - 1 || 512 * c + 8 * lane < dim;
}

// One row of NC vectors; STREAM selects the nontemporal policy.
template <int NC, bool STREAM>
__device__ __forceinline__ void load_row(V8 (&v)[NC], const uint16_t *base, int lane, int dim) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (valid<NC>(c, lane, dim))
      v[c] = STREAM ? load8_stream(base + 512 * c + 8 * lane) : load8(base + 512 * c + 8 * lane);
    else
      v[c] = V8{{0u, 0u, 0u, 0u}};
  }
}

// Modulation rows read by one row only (per-token) are streamed; rows shared
// by a few consecutive rows keep the default policy.
template <int NC>
__device__ __forceinline__ void load_mod_row(V8 (&v)[NC], const uint16_t *base, int lane, int dim,
                                             bool per_token) {
  if (per_token)
    load_row<NC, true>(v, base, lane, dim);
  else
    load_row<NC, false>(v, base, lane, dim);
}

// Keeps the compiler from moving instructions across this point.  Placed
// between a row's statistics and its output loop, it stops the output's
// LDS reads from being hoisted above the reductions, where they would all
// be live at once (more VGPRs, fewer waves per SIMD).
__device__ __forceinline__ void phase_barrier() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ void unpack8(const V8 &v, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = elem(v, j);
}

// ---------------------------------------------------------------------------
// binary32 staging rows in LDS.  Element 512c + 8l + j of a row is component
// j % 4 of float4 (2c + j / 4) * 64 + l: a lane reads the 8 values of its
// chunk c with two ds_read_b128, each covering 64 consecutive float4s across
// the wave (no bank conflicts).  A staged row takes NC * 128 float4s.
// ---------------------------------------------------------------------------
template <int NC>
constexpr int stage_vecs() {
  return NC * 128;
}

// Stores the 8 values of vector v (elements 8v .. 8v + 7).
__device__ __forceinline__ void stage_put(float4 *row, int v, const float (&f)[8]) {
  const int c = v >> 6, l = v & 63;
  row[(2 * c) * 64 + l] = make_float4(f[0], f[1], f[2], f[3]);
  row[(2 * c + 1) * 64 + l] = make_float4(f[4], f[5], f[6], f[7]);
}

__device__ __forceinline__ void stage_get(const float4 *row, int c, int lane, float (&f)[8]) {
  const float4 a = row[(2 * c) * 64 + lane], b = row[(2 * c + 1) * 64 + lane];
  f[0] = a.x;
  f[1] = a.y;
  f[2] = a.z;
  f[3] = a.w;
  f[4] = b.x;
  f[5] = b.y;
  f[6] = b.z;
  f[7] = b.w;
}

// The staging is split in two so that a workgroup's first rows are already
// on their way from HBM while it stages: stage_fetch issues the global loads
// of the vectors this thread converts (vector v = threadIdx.x + i kThreads,
// i < stage_iters), the kernel then issues its first row's loads, and only
// then converts the fetched vectors into LDS (stage_each).
template <int NC>
constexpr int stage_iters() {
  return (NC * 64 + kThreads - 1) / kThreads;
}

template <int NC>
__device__ __forceinline__ void stage_fetch(V8 (&buf)[stage_iters<NC>()], const uint16_t *src,
                                            int dim) {
#pragma unroll
  for (int i = 0; i < stage_iters<NC>(); ++i) {
    const int v = (int)threadIdx.x + i * kThreads;
    if (v < dim / 8)
      buf[i] = load8(src + 8 * v);
    else
      buf[i] = V8{{0u, 0u, 0u, 0u}};
  }
}

// f(i, v) for each fetched vector i of this thread that lies in the row (v
// is its vector index).
template <int NC, class F>
__device__ __forceinline__ void stage_each(int dim, F f) {
#pragma unroll
  for (int i = 0; i < stage_iters<NC>(); ++i) {
    const int v = (int)threadIdx.x + i * kThreads;
    if (v < dim / 8) f(i, v);
  }
}

// Branch-free forms of the loads above, for the loads a staged kernel issues
// before its staging: every load is issued (indexes clamped into the tensor;
// values outside the row are never used, since every consumer checks
// valid()), so the compiler can count the loads still in flight where the
// staging data is needed and wait for those alone.  With a branch among the
// loads it must wait for all of them there (s_waitcnt vmcnt(0)) at the join:
// the workgroup's staging then starts only once its rows have arrived
// instead of while they arrive, which cost RMSNorm-scale 0.9 us and
// RMSNorm-tanh-residual 1.1 us at the Qwen-Image shape.
template <int NC>
__device__ __forceinline__ void stage_fetch_nb(V8 (&buf)[stage_iters<NC>()], const uint16_t *src,
                                               int dim) {
#pragma unroll
  for (int i = 0; i < stage_iters<NC>(); ++i) {
    const int v = (int)threadIdx.x + i * kThreads;
    buf[i] = load8(src + 8 * (v < dim / 8 ? v : dim / 8 - 1));
  }
}

template <int NC, bool STREAM>
__device__ __forceinline__ void load_row_nb(V8 (&v)[NC], const uint16_t *base, int lane,
                                            int dim) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = 512 * c + 8 * lane;
    const int at = (c < NC - 1 || col < dim) ? col : dim - 8;
    v[c] = STREAM ? load8_stream(base + at) : load8(base + at);
  }
}

// ---------------------------------------------------------------------------
// Row runs of this wave.
// ---------------------------------------------------------------------------
struct Span {
  int64_t begin, end;   // the wave's rows [begin, end) (may be empty)
  int64_t m;            // modulation row of the workgroup (staged layout only)
  bool wg_empty;        // the whole workgroup has no rows
};

// Consecutive rows: workgroup b covers rows [4 b rpw, 4 (b + 1) rpw).
__device__ __forceinline__ Span spans(int64_t rows, int64_t rpw) {
  Span s;
  const int64_t wg_first = (int64_t)blockIdx.x * kWavesPerBlock * rpw;
  s.wg_empty = wg_first >= rows;
  s.begin = wg_first + (int64_t)(threadIdx.x >> 6) * rpw;
  s.end = s.begin + rpw < rows ? s.begin + rpw : rows;
  s.m = 0;
  return s;
}

// Per modulation row: workgroup b covers block b % blocks_per_mod of the
// rows of modulation row b / blocks_per_mod; the last block of a modulation
// row may be short (its trailing waves then have no rows).
__device__ __forceinline__ Span mod_spans(int64_t per_mod, int64_t rpw, int64_t blocks_per_mod) {
  Span s;
  s.m = (int64_t)blockIdx.x / blocks_per_mod;
  const int64_t i = (int64_t)blockIdx.x - s.m * blocks_per_mod;
  const int64_t mod_end = (s.m + 1) * per_mod;
  const int64_t wg_first = s.m * per_mod + i * kWavesPerBlock * rpw;
  s.wg_empty = false;                                       // i < blocks_per_mod
  s.begin = wg_first + (int64_t)(threadIdx.x >> 6) * rpw;
  s.end = s.begin + rpw < mod_end ? s.begin + rpw : mod_end;
  return s;
}

// ---------------------------------------------------------------------------
// Launch shapes.
//   One row per wave (four per workgroup) measured fastest for every kernel:
//   at the Wan 720p shape RMSNorm-tanh-residual takes 503 us with one row
//   per wave against 574 us with four, and the Qwen-Image shapes are within
//   noise.  Per-batch modulation (at least one workgroup's worth of rows per
//   modulation row) takes the staged layout: blocks_per_mod workgroups per
//   modulation row, each converting its modulation operands into LDS once.
//   Otherwise the kernels take the split-row layout (dit_split.hpp), except
//   RMSNorm-tanh-residual, whose rows are laid out consecutively, one per
//   wave, each wave loading its row's operands.
// ---------------------------------------------------------------------------

// Staging several binary32 rows stops paying once it limits the workgroups
// per CU; above this LDS size the waves load the operands themselves.
constexpr size_t kMaxStagedLds = 64 * 1024;

struct Shape {
  int64_t rows_per_wave, blocks_per_mod;
  bool staged;
  dim3 grid;
};

// LDS bytes of `rows` binary32 staged rows.
inline size_t stage_bytes(int64_t dim, int rows) {
  return (size_t)rows * (size_t)((dim + 511) / 512) * 128 * sizeof(float4);
}

// staged_rows: binary32 rows the staged layout keeps in LDS (0: the kernel
// never stages; its waves load their modulation rows themselves).
inline Shape row_shape(int64_t rows, int64_t per_mod, int64_t dim, int staged_rows) {
  Shape s;
  s.rows_per_wave = 1;
  const int64_t wg_rows = kWavesPerBlock * s.rows_per_wave;
  s.staged = staged_rows > 0 && per_mod >= wg_rows &&
             stage_bytes(dim, staged_rows) <= kMaxStagedLds;
  const int64_t blocks_per_mod = (per_mod + wg_rows - 1) / wg_rows;
  if (s.staged && rows / per_mod * blocks_per_mod > 0x7FFFFFFF) s.staged = false;
  if (s.staged) {
    s.blocks_per_mod = blocks_per_mod;
    s.grid = dim3((unsigned)(rows / per_mod * blocks_per_mod));
  } else {
    s.blocks_per_mod = 0;
    s.grid = dim3((unsigned)((rows + wg_rows - 1) / wg_rows));
  }
  return s;
}

#define DIT_NC_CASES(X) \
  X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

// Selects the instantiation NC = ceil(dim / 512) through the X macro in scope.
#define DIT_ROW_DISPATCH()                      \
  do {                                          \
    switch ((int)((a.dim + 511) / 512)) {       \
      DIT_NC_CASES(X)                           \
      default: return hipErrorInvalidValue;     \
    }                                           \
    return hipGetLastError();                   \
  } while (0)

// The staged (KT) or unstaged (KF) instantiation, with its LDS bytes.
#define DIT_ROW_LAUNCH(KT, KF, shm_t, shm_f)                        \
  if (sh.staged)                                                    \
    DIT_LAUNCH(KT, sh.grid, dim3(kThreads), shm_t, s, a);           \
  else                                                              \
    DIT_LAUNCH(KF, sh.grid, dim3(kThreads), shm_f, s, a);

}  // namespace dit
