// Device-side helpers and the launch-parameter block shared by the FwPKM
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwpkm {

constexpr int kWave = 64;
constexpr int kKeyBlock = 64;       // smallest key block of the score kernel
constexpr int kTokTile = 16;        // tokens per score workgroup (MFMA N)
constexpr int kGroupWaves = 8;      // waves of one grouping workgroup
constexpr int kSortMaxPairs = 8192; // C*k limit of the in-LDS sort
constexpr int kShortSeg = 16;       // longest segment one update wave sums alone
constexpr int kUpdMaxLists = 3072;  // 3 * units the update kernel can index
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
  int key_block;  // sub-keys per score workgroup (64, 128 or 256)
  int nblk;       // key blocks per half = ceil(n / key_block)
  int P;          // pairs per unit = T * k
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
  // grouping output, per (list, unit) in [3, U, P] arrays; region r of a list
  // owns entries [offset_r, offset_r + its pairs)
  int2* pay;       // sorted (token, coefficient bits) of each list's pairs
  int4* long_rec;  // (row, first pair, pairs, 0) of segments > kShortSeg pairs
  int4* short_rec; // the same for the other segments
  int4* kinds;     // [3, U, regions] (long segments, short segments, offset_r, 0)
  int regions;     // hash regions per (list, unit), a power of two
  int region_bits; // log2(regions)
  int pw;          // floats per row = max(d_v, d_h)
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// (a, ia) strictly precedes (b, ib): smaller value, then smaller index.
__device__ __forceinline__ bool precedes(float a, int ia, float b, int ib) {
  return a < b || (a == b && ia < ib);
}

// ---- cross-lane exchange with lane ^ S, without the LDS permute unit:
// DPP quad permutes for S = 1, 2; row shifts for S = 4; a row rotation for
// S = 8; the gfx950 half-swap instructions for S = 16, 32.  All lanes of the
// wave must be active.
template <int S>
__device__ __forceinline__ int xor_lane(int x) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "stride");
  if constexpr (S == 1) {
    return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);   // row_shl:4
    const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    return (lane_id() & 4) ? dn : up;
  } else if constexpr (S == 8) {
    return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane_id() & 16) ? (int)p[0] : (int)p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane_id() & 32) ? (int)p[0] : (int)p[1];
  }
}
template <int S>
__device__ __forceinline__ float xor_lane(float x) {
  return __int_as_float(xor_lane<S>(__float_as_int(x)));
}
template <int S>
__device__ __forceinline__ double xor_lane(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = xor_lane<S>((int)(b & 0xffffffffll));
  const int hi = xor_lane<S>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Value of lane l (l uniform across the wave); reads the lane even when it
// is inactive.
__device__ __forceinline__ int readlane_i(int x, int l) {
  return __builtin_amdgcn_readlane(x, l);
}
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Butterfly sum over the wave (every lane gets the total, in one fixed order).
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
  x += xor_lane<32>(x);
  x += xor_lane<16>(x);
  x += xor_lane<8>(x);
  x += xor_lane<4>(x);
  x += xor_lane<2>(x);
  x += xor_lane<1>(x);
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) { return wave_sum<double>(x); }

template <int S>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = xor_lane<S>(v);
  const int oi = xor_lane<S>(i);
  if (precedes(ov, oi, v, i)) { v = ov; i = oi; }
}

// Wave-wide best (value, index) under `precedes`; every lane gets it.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<32>(v, i);
  best_step<16>(v, i);
  best_step<8>(v, i);
  best_step<4>(v, i);
  best_step<2>(v, i);
  best_step<1>(v, i);
}

// One compare-exchange of a bitonic network with partner lane ^ S.
template <int S>
__device__ __forceinline__ void cas_step(float& v, int& i, bool ascending) {
  const float ov = xor_lane<S>(v);
  const int oi = xor_lane<S>(i);
  const bool lower = (lane_id() & S) == 0;
  const bool want_better = (lower == ascending);
  const bool self_better = precedes(v, i, ov, oi);
  if (want_better != self_better && (v != ov || i != oi)) { v = ov; i = oi; }
}

template <int SIZE, int S>
__device__ __forceinline__ void bitonic_merge_steps(float& v, int& i) {
  const bool ascending = SIZE == kWave || (lane_id() & SIZE) == 0;
  cas_step<S>(v, i, ascending);
  if constexpr (S > 1) bitonic_merge_steps<SIZE, S / 2>(v, i);
}

template <int SIZE>
__device__ __forceinline__ void bitonic_stages(float& v, int& i) {
  if constexpr (SIZE > 2) bitonic_stages<SIZE / 2>(v, i);
  bitonic_merge_steps<SIZE, SIZE / 2>(v, i);
}

// Bitonic sort of one (value, index) per lane across the wave, best first.
__device__ __forceinline__ void wave_bitonic_sort(float& v, int& i) { bitonic_stages<kWave>(v, i); }

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
