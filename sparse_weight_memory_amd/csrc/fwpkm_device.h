// Device-side helpers and the launch-parameter block shared by the FwPKM
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwpkm {

constexpr int kWave = 64;
constexpr int kKeyBlock = 256;      // sub-keys scored by one score workgroup
constexpr int kTokTile = 16;        // tokens per score workgroup (MFMA N)
constexpr int kSortThreads = 1024;  // threads of one sort workgroup
constexpr int kSortMaxPairs = 8192; // C*k limit of the in-LDS sort
constexpr int kDigitBits = 6;       // radix digit of the sort
constexpr int kUpdWaves = 4;        // waves per update workgroup
#define FWPKM_MAX_HALF_DIM 1024     // largest d_h the score kernel stages

// Invalid entries: they order after every real candidate.
constexpr int kNoIndex = 0x7fffffff;

// Everything a chunk's kernels need, passed by value.
struct ChunkArgs {
  // sizes
  int n;          // sub-keys per half
  int half;       // d_h = d_qk / 2
  int dqk;
  int dv;
  int k;          // top-k
  int T;          // tokens of this call
  int H;          // heads
  int U;          // units = batch * H
  int nblk;       // key blocks per half = ceil(n / kKeyBlock)
  int P;          // pairs per unit = T * k
  int key_bits_v; // bits of a V key (slot)
  int key_bits_k; // bits of a K key (row, with the n marker)
  int mode;       // 0 IDW, 1 dot
  float eps;
  float lr;
  // inputs
  const float* q;   // [B, T, H, dqk]
  const float* y;   // [B, T, H, dv]
  // state (tables the chunk reads; the update writes the same tables)
  float* k1;
  float* k2;
  float* v;
  int64_t stride_k;   // elements between sequences
  int64_t stride_v;
  // outputs
  float* retrieved;   // [B, T, H, dv]
  int* out_slots;     // nullable [B, T, H, k]
  float* out_weights; // nullable [B, T, H, k]
  // workspace
  float* half_o;   // [U, T, 2, nblk, k] ordering keys of per-half candidates
  int* half_i;     // [U, T, 2, nblk, k] their sub-key indices
  float* qnorm;    // [U, T, 2]
  float* sel_w;    // [U, P] weight of pair p = t*k + m
  float* g;        // [U, T, dv] retrieved - target
  int* keys;       // [3, U, P] V slot | K1 row (n = none) | K2 row (n = none)
  float* coef;     // [2, U, P] merged key coefficient of a K1 / K2 pair
  int* sorted;     // [3, U, P] pair indices ordered by key (stable)
  int* seg_start;  // [3, U, P + 1] first sorted position of each segment
  int* nseg;       // [3, U] segments per list
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// (a, ia) strictly precedes (b, ib): smaller value, then smaller index.
__device__ __forceinline__ bool precedes(float a, int ia, float b, int ib) {
  return a < b || (a == b && ia < ib);
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int x, int m) { return __shfl_xor(x, m, kWave); }

// Value of lane l (l uniform across the wave); reads the lane even when it
// is inactive.
__device__ __forceinline__ int readlane_i(int x, int l) {
  return __builtin_amdgcn_readlane(x, l);
}
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) x += shfl_xor_f(x, m);
  return x;
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// Wave-wide best (value, index) under `precedes`; every lane gets it.
__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) {
    float ov = shfl_xor_f(v, m);
    int oi = shfl_xor_i(i, m);
    if (precedes(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// Bitonic sort of one (value, index) per lane across the wave, best first.
__device__ __forceinline__ void wave_bitonic_sort(float& v, int& i) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      float ov = shfl_xor_f(v, stride);
      int oi = shfl_xor_i(i, stride);
      const bool ascending = (lane & size) == 0 || size == kWave;
      const bool lower = (lane & stride) == 0;
      const bool want_better = (lower == ascending);
      const bool self_better = precedes(v, i, ov, oi);
      if (want_better != self_better && (v != ov || i != oi)) { v = ov; i = oi; }
    }
  }
}

// k rounds of wave-wide argmin over J candidates per lane; lane r < k ends
// up holding the r-th best (value, index).  Removed or empty entries are
// (+inf, kNoIndex) and order after every real candidate.
template <int J>
__device__ __forceinline__ void wave_select_k(float (&cv)[J], int (&ci)[J], int k,
                                              float& mine_v, int& mine_i) {
  const int lane = lane_id();
  mine_v = __builtin_inff();
  mine_i = kNoIndex;
  for (int round = 0; round < k; ++round) {
    float bv = cv[0];
    int bi = ci[0];
#pragma unroll
    for (int j = 1; j < J; ++j)
      if (precedes(cv[j], ci[j], bv, bi)) { bv = cv[j]; bi = ci[j]; }
    wave_best(bv, bi);
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (ci[j] == bi && cv[j] == bv) { cv[j] = __builtin_inff(); ci[j] = kNoIndex; }
    if (lane == round) { mine_v = bv; mine_i = bi; }
  }
}

// Sanitise an ordering key: NaN orders last.
__device__ __forceinline__ float order_key(float x) {
  return (x != x) ? __builtin_inff() : x;
}

}  // namespace fwpkm
