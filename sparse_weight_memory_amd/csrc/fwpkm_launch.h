// Host-side launchers of the FwPKM kernels (one per kernel family).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "fwpkm_device.h"

namespace fwpkm {

// Optional start/stop events stamped by the kernel dispatch itself
// (hipExtLaunchKernelGGL), so the measured time is the kernel's own.
struct LaunchTiming {
  hipEvent_t beg = nullptr;
  hipEvent_t end = nullptr;
};

template <typename K, typename... Args>
inline hipError_t fw_launch(K kernel, dim3 grid, dim3 block, uint32_t smem, hipStream_t s,
                            const LaunchTiming* tm, Args... args) {
  if (tm)
    hipExtLaunchKernelGGL(kernel, grid, block, smem, s, tm->beg, tm->end, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, smem, s, args...);
  return hipGetLastError();
}

// KA: score GEMM + per-half top-k per key block.  score_key_block() picks the
// block (64, 128 or 256 keys) for a chunk shape.
int score_key_block(int units, int tokens, int n);
hipError_t launch_ka(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm);

// KB: Cartesian top-k, softmax weights, value gather-reduce and, when
// `write`, the fast-weight backward that emits the (row, pair) lists.
hipError_t launch_kb(const ChunkArgs& a, bool write, hipStream_t s, const LaunchTiming* tm);

// KC: per (region, list, unit) stable radix sort of the pair lists, segment
// records by length.  group_regions() picks the hash regions per list.
int group_regions(int units);
size_t kc_smem_bytes(int P);
hipError_t launch_kc(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm);

// KE: marginal-entropy addressing loss (only with addr_weight != 0):
// softmax statistics, marginal usage and dL/ds coefficients per (unit,
// half) (three kernels, timed as one span), the key-gradient contraction,
// and the key step after the update.
hipError_t launch_ke_stats(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm);
hipError_t launch_ke_grad(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm);
hipError_t launch_ke_apply(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm);

// KF: the sequence-level layer: projection GEMM with lookahead targets (and
// the last-token prep, timed as one span), then the gated output.
hipError_t launch_kf_project(const SeqArgs& s, hipStream_t st, const LaunchTiming* tm);
hipError_t launch_kf_gate(const SeqArgs& s, hipStream_t st, const LaunchTiming* tm);

// KD: per segment mean gradient and in-place SGD on V, K1 and K2 rows.
// When kd_fuses_grouping(a) (at most 2048 pairs per unit) the update kernel
// groups the rows itself and KC must not be launched.
bool kd_fuses_grouping(const ChunkArgs& a);
hipError_t launch_kd(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm);

}  // namespace fwpkm
