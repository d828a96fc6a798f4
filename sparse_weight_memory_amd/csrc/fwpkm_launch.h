// Host-side launchers of the FwPKM kernels (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "fwpkm_device.h"

namespace fwpkm {

// KA: score GEMM + per-half top-k per 256-key block.
size_t ka_smem_bytes(int half);
hipError_t launch_ka(const ChunkArgs& a, hipStream_t s);

// KB: Cartesian top-k, softmax weights, value gather-reduce and, when
// `write`, the fast-weight backward that emits the (row, pair) lists.
hipError_t launch_kb(const ChunkArgs& a, bool write, hipStream_t s);

// KC: per (unit, list) stable radix sort of the pair lists + segments.
size_t kc_smem_bytes(int P);
hipError_t launch_kc(const ChunkArgs& a, hipStream_t s);

// KD: per segment mean gradient and in-place SGD on V, K1 and K2 rows.
hipError_t launch_kd(const ChunkArgs& a, hipStream_t s);

}  // namespace fwpkm
