// Device-side helpers and the launch-parameter block shared by the FwPKM
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fwpkm {

constexpr int kWave = 64;
constexpr int kKeyBlock = 64;       // smallest key block of the score kernel
constexpr int kTokTile = 16;        // tokens per score workgroup (MFMA N)
constexpr int kReadTokensMax = 4;  // tokens (one wave each) per read workgroup, at most
constexpr int kAddrPad = 256;   // score-row pitch multiple of the addressing loss (4 loads per lane)
constexpr int kGroupWaves = 8;      // waves of one grouping workgroup
constexpr int kSortMaxPairs = 8192; // C*k limit of the in-LDS sort
constexpr int kUpdMaxLists = 3072;  // 3 * units (lists) a chunk may carry
#define FWPKM_MAX_HALF_DIM 1024     // largest d_h the score kernel stages

// Invalid entries: they order after every real candidate.
constexpr int kNoIndex = 0x7fffffff;

// Checked builds (FWPKM_DEVICE_CHECKS=1): the kernels test the invariants the
// indexing rests on and set a bit in ChunkArgs::check for every one that
// fails; the host reads the word after the call.  Off by default, where the
// tests compile away.
#ifndef FWPKM_DEVICE_CHECKS
#define FWPKM_DEVICE_CHECKS 0
#endif
enum DeviceCheck : unsigned int {
  kChkHalfIndex = 1u << 0,    // a per-half candidate's sub-key index is >= n
  kChkCandidates = 1u << 1,   // fewer than k Cartesian candidates for a token
  kChkSlot = 1u << 2,         // a selected slot is outside [0, N)
  kChkDistinct = 1u << 3,     // a token selected one slot twice
  kChkWeight = 1u << 4,       // a selection weight is not finite or outside [0, 1]
  kChkEntry = 1u << 5,        // a grouped entry's row or token is out of range, or not its pair's row
  kChkCapacity = 1u << 6,     // an update batch overflows its LDS lists
  kChkOrder = 1u << 7,        // grouped entries are not sorted by row
};
constexpr int kNumDeviceChecks = 8;

// Everything a chunk's kernels need, passed by value.
// Division by a divisor d >= 1 fixed for a launch, for dividends 0 <= x < 2^31:
// x / d = (umulhi(x, m) + x) >> l with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1 (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994).  The host derives (m, l)
// once; in a kernel the quotient costs three scalar instructions where a
// runtime integer division costs about thirty, and the scalar unit is shared
// by every wave of a compute unit.
struct FastDiv {
  unsigned int m;
  int l;
};

inline FastDiv make_fastdiv(int d) {
  int l = 0;
  while ((1ll << l) < (long long)d) ++l;
  const unsigned long long m = ((1ull << 32) * ((1ull << l) - (unsigned long long)d)) / (unsigned long long)d + 1;
  return FastDiv{(unsigned int)m, l};
}

__host__ __device__ __forceinline__ int fast_div(int x, FastDiv f) {
#if __HIP_DEVICE_COMPILE__
  const unsigned int hi = __umulhi((unsigned int)x, f.m);
#else
  const unsigned int hi = (unsigned int)(((unsigned long long)(unsigned int)x * f.m) >> 32);
#endif
  return (int)((hi + (unsigned int)x) >> f.l);
}

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
  const float* tw;  // nullable [B, T, H] token-importance weights (null = all 1)
  // state (tables the chunk reads; the update writes the same tables)
  float* k1;
  float* k2;
  float* v;
  int64_t stride_k;   // elements between sequences
  int64_t stride_v;
  // outputs
  float* retrieved;   // [B, ., H, dv]: row (b, t, h) at b * out_rows_b + t * H + h
  int64_t out_rows_b; // (token, head) rows between sequences in retrieved / out_slots /
                      // out_weights: T * H for a chunk call, S * H inside a sequence
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
  int* ent_row;    // each list's kept entries' rows, sorted by row (stable)
  int2* ent_tw;    // their (token, weight bits): V softmax weight / K coefficient
  int4* kinds;     // [3, U, regions] (0, 0, offset_r, entries)
  int regions;     // hash regions per (list, unit), a power of two
  int region_bits; // log2(regions)
  int pw;          // floats per row = max(d_v, d_h)
  int npr;         // Cartesian candidates (i, j) with (i+1)(j+1) <= k: sum_i floor(k/(i+1))
  // marginal-entropy addressing loss (addr_s == nullptr: off)
  float addr_weight;   // lambda
  float* addr_s;       // [U, 2, T, addr_np] ordering keys of every (token, sub-key); later dL/ds coefficients
  int addr_np;         // row pitch of addr_s: n rounded up to kAddrPad (pad columns hold no data)
  float* addr_dk;      // [U, 2, n, d_h] addressing gradient of each key row
  float* addr_tok;     // [U, 2, T, 2] per token: softmax shift m (dot) and 1 / softmax sum
  float* addr_ell;     // [U, 2, n] log marginal usage of each sub-key
  // score-kernel geometry, derived on the host by its launcher
  int ka_ntt;          // 16-token tiles = ceil(T / 16)
  int ka_nkt_log2;     // log2(key_block / 16): key tiles per block
  int ka_share;        // dims of d_h per dim share of a wave
  FastDiv ka_div_ntt;  // x / ka_ntt
  FastDiv ka_div_nblk; // x / nblk
  // divisors of the work-item decompositions, derived on the host by every
  // launcher that uses them (with_divisors)
  FastDiv div_H;       // x / H
  FastDiv div_U;       // x / U
  FastDiv div_upx;     // x / (U / 8): units per XCD
  // read-kernel geometry, derived on the host by its launcher
  int kb_tpw;          // tokens (one wave each) per read workgroup
  int kb_nbx;          // read workgroups per unit = ceil(T / kb_tpw)
  FastDiv kb_div_nbx;  // x / kb_nbx
  // update-kernel geometry, derived on the host by its launcher: column
  // slices, kd_sv of them per V row and kd_sk per K row; kd_gv hash groups
  // of rows per value list and kd_gk per sub-key list
  int kd_sv;
  int kd_sk;
  int kd_gv;
  int kd_gk;
  int kd_pu;           // workgroups per unit: kd_sv kd_gv + 2 kd_sk kd_gk
  FastDiv kd_div_pu;   // x / kd_pu
  FastDiv kd_div_gv;   // x / kd_gv
  FastDiv kd_div_gk;   // x / kd_gk
  FastDiv kd_div_kl;   // x / (kd_sk kd_gk): workgroups per sub-key list
  unsigned int* check; // one word of DeviceCheck bits (checked builds)
};

// Sets `bit` in the check word when `ok` is false (checked builds only).
__device__ __forceinline__ void device_check(const ChunkArgs& a, bool ok, unsigned int bit) {
#if FWPKM_DEVICE_CHECKS
  if (!ok) atomicOr(a.check, bit);
#else
  (void)a; (void)ok; (void)bit;
#endif
}

// `a` with the decomposition divisors filled in
inline ChunkArgs with_divisors(const ChunkArgs& a) {
  ChunkArgs g = a;
  g.div_H = make_fastdiv(a.H > 1 ? a.H : 1);
  g.div_U = make_fastdiv(a.U > 1 ? a.U : 1);
  g.div_upx = make_fastdiv(a.U / 8 > 1 ? a.U / 8 : 1);
  return g;
}

// The sequence-level layer around the chunk step (queries/values projected
// from model-width tokens, lookahead targets, gated output).
struct SeqArgs {
  const float* x;       // [B, S, D] tokens, D = H * dv
  const float* w_in;    // [Nq + Nv, D]: query rows (head-major), then value rows
  const float* w_gate;  // [H, D]
  const float* b_gate;  // nullable [H]
  float* q_all;         // chunk-major queries: chunk c holds [B, Cc, H, dqk]
  float* y_all;         // chunk-major targets (value of the next token): [B, Cc, H, dv]
  float* tw_last;       // [B, C_last, H] token weights of the last chunk
  float* out;           // [B, S, D]: memory reads, then the gated output in place
  int B, S, D, H, dqk, dv;
  int C;                // chunk size (the last chunk may be shorter)
  int Nq, Nv;           // H * dqk, H * dv
};

// Row of token (b, t) in the chunk-major layout: chunk c = t / C starts after
// c full chunks of B * C rows and holds B sequences of Cc tokens each.
__device__ __forceinline__ int64_t seq_chunk_row(const SeqArgs& s, int b, int t) {
  const int c = t / s.C, tt = t - c * s.C;
  const int cc = min(s.C, s.S - c * s.C);
  return (int64_t)c * s.B * s.C + (int64_t)b * cc + tt;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Bits needed to write x >= 0 (0 for x = 0): one count-leading-zeros.  A
// loop over the bits would run on the compute unit's one scalar unit once
// per wave.
__device__ __forceinline__ int bit_length(int x) { return 32 - __clz(x); }

// Token of pair p = t*k + m without an integer divide: (p + 1/2) / k lies at
// least 1/(2k) >= 1/64 away from an integer, relative 2e-6 at p < 8192, far
// above the reciprocal's error.
__device__ __forceinline__ int token_of(int p, int k) {
  return (int)(((float)p + 0.5f) * __builtin_amdgcn_rcpf((float)k));
}

// Units and XCDs.  Workgroup i of every launch runs on XCD i % 8 (the
// dispatcher deals workgroups to the eight XCDs in turn), each XCD has its
// own L2, and that L2 keeps what one kernel wrote for the next.  When the
// unit count is a multiple of 8, the score kernel's layout runs unit u on XCD
// u / (U / 8); kernels whose work items are unit-major follow it, so a unit's
// candidate lists, pair lists and g rows are read back from the L2 that
// holds them.  Returns the work item of workgroup `wg` for a grid of exactly
// units * per_unit workgroups (the identity when units % 8 != 0).
constexpr int kXcds = 8;
__device__ __forceinline__ int unit_affine_item(int wg, int units, int per_unit) {
  if (units % kXcds != 0) return wg;
  return (wg % kXcds) * (units / kXcds) * per_unit + wg / kXcds;
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

// Inclusive prefix sum across the wave: DPP row shifts within each row of 16
// lanes, then the lower rows' totals by readlane.  All lanes must be active.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int r0 = readlane_i(x, 15), r1 = readlane_i(x, 31), r2 = readlane_i(x, 47);
  const int row = lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Workgroup barrier that orders LDS traffic only: each wave waits for its own
// LDS operations, then for the other waves.  __syncthreads() first waits for
// every global load the wave has in flight as well, so a phase that works
// in LDS while a later phase's global loads travel uses this one.  It makes
// no global memory written before it visible to other waves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// All ones if ok, else zero, through an empty asm: AND-ing a loaded value
// with it masks the value without letting the compiler turn the mask into a
// select, and the select into a branch around the load (every such branch
// waits for its load alone).
__device__ __forceinline__ unsigned int opaque_mask(bool ok) {
  unsigned int m = ok ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return m;
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

// ---- packed sort keys.  A (value, index) candidate packs into one 64-bit
// integer whose unsigned order is the (value asc, index asc) order of
// `precedes`: the value's IEEE bits, made monotone (negative values have all
// bits flipped, the others only the sign bit), in the high word and the
// index in the low word.  -0 is folded to +0 first, so the two zeros compare
// equal as they do as floats; values must not be NaN (see order_key).  The
// empty candidate (+inf, kNoIndex) orders after every real one.
typedef unsigned long long skey;

__device__ __forceinline__ skey pack_key(float v, int i) {
  unsigned int b = __float_as_uint(v == 0.0f ? 0.0f : v);
  b ^= (b & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
  return ((skey)b << 32) | (unsigned int)i;
}
__device__ __forceinline__ float key_value(skey x) {
  unsigned int b = (unsigned int)(x >> 32);
  b ^= (b & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu;
  return __uint_as_float(b);
}
__device__ __forceinline__ int key_index(skey x) { return (int)(unsigned int)x; }
constexpr skey kEmptyKey = 0xFF800000ull << 32 | 0x7fffffffull;   // pack_key(+inf, kNoIndex)

template <int S>
__device__ __forceinline__ skey xor_lane(skey x) {
  const unsigned int lo = (unsigned int)xor_lane<S>((int)(unsigned int)x);
  const unsigned int hi = (unsigned int)xor_lane<S>((int)(unsigned int)(x >> 32));
  return ((skey)hi << 32) | lo;
}
__device__ __forceinline__ skey readlane_k(skey x, int l) {
  const unsigned int lo = (unsigned int)__builtin_amdgcn_readlane((int)(unsigned int)x, l);
  const unsigned int hi = (unsigned int)__builtin_amdgcn_readlane((int)(unsigned int)(x >> 32), l);
  return ((skey)hi << 32) | lo;
}

// One compare-exchange of a bitonic network on packed keys, partner lane ^ S:
// the lane keeps the smaller key when (it is the lower lane) == ascending.
template <int S>
__device__ __forceinline__ void cas_key(skey& x, bool ascending) {
  const skey o = xor_lane<S>(x);
  const bool keep_min = ((lane_id() & S) == 0) == ascending;
  x = ((o < x) == keep_min) ? o : x;
}

template <int SIZE, int GROUP, int S>
__device__ __forceinline__ void key_merge_steps(skey& x) {
  const bool ascending = SIZE == GROUP || (lane_id() & SIZE) == 0;
  cas_key<S>(x, ascending);
  if constexpr (S > 1) key_merge_steps<SIZE, GROUP, S / 2>(x);
}
template <int SIZE, int GROUP>
__device__ __forceinline__ void key_stages(skey& x) {
  if constexpr (SIZE > 2) key_stages<SIZE / 2, GROUP>(x);
  key_merge_steps<SIZE, GROUP, SIZE / 2>(x);
}

// Smallest packed key of the wave, in every lane.
__device__ __forceinline__ skey min_lanes(skey x) {
  skey o;
  o = xor_lane<32>(x); x = o < x ? o : x;
  o = xor_lane<16>(x); x = o < x ? o : x;
  o = xor_lane<8>(x);  x = o < x ? o : x;
  o = xor_lane<4>(x);  x = o < x ? o : x;
  o = xor_lane<2>(x);  x = o < x ? o : x;
  o = xor_lane<1>(x);  x = o < x ? o : x;
  return x;
}

// Bitonic sort of one packed key per lane within every aligned group of
// GROUP lanes (8, 16, 32 or 64), ascending in each group.  All lanes active.
template <int GROUP>
__device__ __forceinline__ void sort_keys(skey& x) {
  static_assert(GROUP == 8 || GROUP == 16 || GROUP == 32 || GROUP == 64, "group");
  key_stages<GROUP, GROUP>(x);
}

// Sanitise an ordering key: NaN orders last.
__device__ __forceinline__ float order_key(float x) {
  return (x != x) ? __builtin_inff() : x;
}

}  // namespace fwpkm
