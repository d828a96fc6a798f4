// KD: per-row mean gradient and in-place SGD step on the touched V, K1 and
// K2 rows.
//
// For a row r touched by the n_r tokens of its segment (pairs in ascending
// token order):
//   V row   theta_r <- theta_r - lr * (1/n_r) sum_p w_p g_{t_p}
//   K1 row  IDW: theta_r <- theta_r - lr * (1/n_r) sum_p c_p (q1_{t_p} - theta_r)
//           dot: theta_r <- theta_r - lr * (1/n_r) sum_p c_p q1_{t_p}
//   K2 row  likewise with q2.
// All gradients are taken at the chunk's starting weights: every (row,
// column) is read and then written by one wave of one workgroup, so
// updating in place is exact.
// [agifrontier tutorial "Fast-weight Product Key Memory", update equation
// theta' = theta - eta grad L_MSE; gist.science summary, section 2: Key and
// Value matrices updated online, gradients of a slot used several times in a
// chunk averaged; sciencestack.ai contents: no gradient clipping]
//
// Work distribution.  A row's gradient is a sum over its tokens' data rows
// (g_t for V, a query half for K), and a row touched by many tokens (the
// common case with clustered queries) would stream all of those rows through
// one compute unit.  Instead every list is cut into column slices of SW
// floats: a workgroup owns (unit, list, column slice, group of hash
// regions), stages that slice of every token's data row in LDS once, and
// sums each of its rows' pairs from LDS.  A hot row is thus spread over as
// many compute units as its list has slices, and each pair costs an LDS read
// instead of a dependent global load.
//
// Grouping.  With at most kKdEntCap pairs per unit (kd_write), the
// workgroup groups its rows itself: it loads the list's row keys and
// weights (coefficients) and orders the rows of its hash group by row, a
// row's pairs in ascending token order.  Rows of up to 16 bits are first
// renamed to their rank among the group's distinct rows (a bitmap of the
// rows present); with at most 256 ranks and 256 tokens, every rank's tokens
// are set as bits of a mask in LDS, and an entry's place is a popcount of
// the masks (ranks below its own, tokens below its own in its rank), which
// also gives the segments and their tables.  Otherwise the rows are kept in
// pair order and sorted stably with an LSD radix sort in LDS (8-bit digits,
// ballot ranking).  The grouping is repeated by the column slices of one group, which is
// cheaper than a separate grouping launch and its dependent global rounds;
// value and sub-key lists take separate numbers of hash groups, chosen to
// even out the workgroups' work.  Larger chunks (kd_update) read the grouping kernel's
// output instead: per (list, unit), the kept entries sorted by row, each
// with its token and weight, regions one after another, so a group of
// consecutive regions is one contiguous run of entries, taken in batches
// cut at segment heads.  Either way the segments (runs of one row) are
// found here.  Work items: a segment of at most SW/4 pairs is short, and
// 256/SW of them share a wave pass, one per pair group; a longer segment is
// cut into kKdPiece-pair pieces, each summed by a whole wave (the pieces'
// partial sums meet in LDS and are added in piece order).  Inside a
// wave the lanes form SW/4 float4 columns times 256/SW pair groups; lane l
// holds the token and weight of one pair, pair group g sums pairs g,
// g + groups, ... as DPP broadcasts hand them over (only as many steps as the
// item needs), and a fixed butterfly adds the groups.  Every sum runs in
// one fixed order, results do not depend on scheduling, and no atomic
// operation touches a sum (the only atomics set bits of the row bitmap and
// of the per-rank token masks, whose values do not depend on their order).

#include <algorithm>

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kKdWaves = 16;                    // waves of an update workgroup
constexpr int kKdThreads = kKdWaves * kWave;
constexpr int kKdDataBytes = 64 * 1024;         // a column slice of every token's data row
constexpr int kKdEntCap = 2048;                 // entries (pairs) staged at a time
constexpr int kKdPer = kKdEntCap / kKdThreads;  // entries per thread
constexpr int kKdPiece = kWave;                 // pairs one wave sums; longer segments are cut
constexpr int kKdMaxLong = 2 * kKdEntCap / kKdPiece;   // pieces of long segments per batch
constexpr int kKdMaxPieces = 1023;              // pieces of a batch (segments of > 4 pairs)
static_assert(kKdEntCap / 5 + kKdMaxLong <= kKdMaxPieces, "piece count fits its field");
constexpr int kKdPrefetch = 2;                  // old-row float4 prefetched per lane per round
static_assert(kKdPer * kKdThreads == kKdEntCap, "whole entries per thread");

// LDS layout (byte offsets) for chunks of T tokens and slices of SW floats.
// The data slice, the one part whose size depends on T, comes last, so every
// other offset is a constant the compiler folds (a runtime layout cost each
// of the 16 waves ~25 instructions on the compute unit's one scalar unit).
struct KdLds {
  int dat, ent_t, ent_w, ent_row, seg_beg, seg_item, short_seg, items, part, part_c, long_seg, red, total;
};
__host__ __device__ constexpr int kd_align(int x) { return (x + 15) & ~15; }
__host__ __device__ constexpr KdLds kd_lds_layout(int T, int SW) {
  KdLds L{};
  int o = 0;
  L.ent_t = o;    o = kd_align(o + kKdEntCap * 4);
  L.ent_w = o;    o = kd_align(o + kKdEntCap * 4);
  L.ent_row = o;  o = kd_align(o + (kKdEntCap + 1) * 4);         // + the row after the batch
  L.seg_beg = o;  o = kd_align(o + (kKdEntCap + 1) * 4);         // segment starts, then the end
  L.seg_item = o; o = kd_align(o + kKdEntCap * 4);               // short index | piece << 12 | slot << 22
  L.short_seg = o; o = kd_align(o + kKdEntCap * 4);              // short segments in order
  L.items = o;    o = kd_align(o + kKdMaxPieces * 4);            // pieces of longer segments
  L.part = o;     o = kd_align(o + kKdMaxLong * (SW / 4) * 16);  // partial sums of long pieces
  L.part_c = o;   o = kd_align(o + kKdMaxLong * 4);
  L.long_seg = o; o = kd_align(o + kKdMaxLong * 4);
  L.red = o;      o = kd_align(o + 4 * kKdWaves * 4);
  L.dat = o;      o = kd_align(o + T * (SW / 4 + 1) * 16);        // [T][SW/4 + 1] float4 (padded rows)
  L.total = o;
  return L;
}

// Exclusive scan of one int per thread over the block; *total = the sum.
// `red` (kKdWaves ints) must not be written again before the caller's next
// barrier.
template <bool kLdsOnly = false>
__device__ __forceinline__ int kd_block_scan(int x, int* red, int* total) {
  const int wave = threadIdx.x / kWave;
  const int incl = wave_inclusive_scan(x);
  if (lane_id() == kWave - 1) red[wave] = incl;
  if constexpr (kLdsOnly) lds_barrier(); else __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kKdWaves; ++w) {
    const int t = red[w];
    base += w < wave ? t : 0;
    sum += t;
  }
  *total = sum;
  return base + incl - x;
}

__device__ __forceinline__ float4 f4_fma(float w, float4 x, float4 acc) {
  acc.x = fmaf(w, x.x, acc.x); acc.y = fmaf(w, x.y, acc.y);
  acc.z = fmaf(w, x.z, acc.z); acc.w = fmaf(w, x.w, acc.w);
  return acc;
}

__device__ __forceinline__ float4 f4_add(float4 x, float4 y) {
  return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
}

template <int S>
__device__ __forceinline__ float4 f4_xor(float4 v) {
  return make_float4(xor_lane<S>(v.x), xor_lane<S>(v.y), xor_lane<S>(v.z), xor_lane<S>(v.w));
}

// Sum over the pair groups (lane bits from log2(L4) up): a fixed butterfly,
// every lane receives the total.  All lanes active.
template <int L4>
__device__ __forceinline__ void pair_group_sum(float4& acc, float& cs) {
  if constexpr (L4 <= 4) { acc = f4_add(acc, f4_xor<4>(acc)); cs += xor_lane<4>(cs); }
  if constexpr (L4 <= 8) { acc = f4_add(acc, f4_xor<8>(acc)); cs += xor_lane<8>(cs); }
  if constexpr (L4 <= 16) { acc = f4_add(acc, f4_xor<16>(acc)); cs += xor_lane<16>(cs); }
  acc = f4_add(acc, f4_xor<32>(acc));
  cs += xor_lane<32>(cs);
}

// Lane (lane & ~(L4 - 1)) + S's value, for every lane: DPP broadcasts within
// quads (L4 = 4) or rows of 16 (L4 = 16; two of them for halves, L4 = 8).
template <int L4, int S>
__device__ __forceinline__ int group_bcast(int x) {
  static_assert(S >= 0 && S < L4, "step");
  if constexpr (L4 == 4) {
    return __builtin_amdgcn_update_dpp(0, x, S * 0x55, 0xF, 0xF, false);         // quad_perm [S,S,S,S]
  } else if constexpr (L4 == 16) {
    return __builtin_amdgcn_update_dpp(0, x, 0x150 + S, 0xF, 0xF, false);        // row_newbcast:S
  } else {
    const int lo = __builtin_amdgcn_update_dpp(0, x, 0x150 + S, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, x, 0x150 + 8 + S, 0xF, 0xF, false);
    return (lane_id() & 8) ? hi : lo;
  }
}

// Steps S, S+1, ... < steps of an item, four at a time (their LDS reads go
// out together; a step past the item's pairs adds weight 0): step s hands
// pair group g its pair held by lane g * L4 + s (pair s * groups + g).
// `steps` is wave-uniform, in a scalar register.
template <int L4, int S>
__device__ __forceinline__ void sum_steps(int steps, int my_t, int my_w, const float4* dat, int c4,
                                          float4& acc, float& cs) {
  if constexpr (S < L4) {
    static_assert(L4 % 4 == 0, "whole batches of four steps");
    if (S >= steps) return;
    const int t[4] = {group_bcast<L4, S>(my_t), group_bcast<L4, S + 1>(my_t),
                      group_bcast<L4, S + 2>(my_t), group_bcast<L4, S + 3>(my_t)};
    const float w[4] = {__int_as_float(group_bcast<L4, S>(my_w)),
                        __int_as_float(group_bcast<L4, S + 1>(my_w)),
                        __int_as_float(group_bcast<L4, S + 2>(my_w)),
                        __int_as_float(group_bcast<L4, S + 3>(my_w))};
    float4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = dat[t[i] * (L4 + 1) + c4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = f4_fma(w[i], x[i], acc);
      cs += w[i];
    }
    sum_steps<L4, S + 4>(steps, my_t, my_w, dat, c4, acc, cs);
  }
}


// Radix digit ranking: lanes of this wave holding the same 8-bit digit
// (among `valid` lanes).
__device__ __forceinline__ unsigned long long digit_peers(int d, bool valid) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const unsigned long long on = __ballot((d >> bit) & 1);
    peers &= ((d >> bit) & 1) ? on : ~on;
  }
  return peers;
}

__device__ __forceinline__ unsigned long long lanes_below() {
  return (1ull << lane_id()) - 1ull;
}

// Hash group of a row among 2^bits: multiplicative (Fibonacci) hashing, so
// rows that many tokens share spread over the groups.
__device__ __forceinline__ int hash_group(int row, int groups) {
  // multiply-range reduction of the 32-bit hash: for 2^b groups, its top b bits
  return (int)(((unsigned long long)((unsigned)row * 0x9E3779B1u) * (unsigned)groups) >> 32);
}

// Which (unit, list, column slice, hash group) an update workgroup owns.
// Per unit: value-row slices times kd_gv groups, then K1's and K2's slices
// times kd_gk groups each; the groups of a slice are adjacent.
struct KdWho {
  int u, list, slice, grp, ngrp, b, hh, width4, col4;
};

__device__ __forceinline__ KdWho kd_who(const ChunkArgs& a, int L4) {
  KdWho w;
  const int item = unit_affine_item(blockIdx.x, a.U, a.kd_pu);
  w.u = fast_div(item, a.kd_div_pu);
  const int rest = item - w.u * a.kd_pu;
  const int nv = a.kd_sv * a.kd_gv;
  if (rest < nv) {
    w.list = 0;
    w.slice = fast_div(rest, a.kd_div_gv);
    w.grp = rest - w.slice * a.kd_gv;
    w.ngrp = a.kd_gv;
  } else {
    const int r2 = rest - nv;
    const int hk = fast_div(r2, a.kd_div_kl);          // / (kd_sk * kd_gk)
    const int r3 = r2 - hk * a.kd_sk * a.kd_gk;
    w.list = 1 + hk;
    w.slice = fast_div(r3, a.kd_div_gk);
    w.grp = r3 - w.slice * a.kd_gk;
    w.ngrp = a.kd_gk;
  }
  w.width4 = (w.list == 0 ? a.dv : a.half) >> 2;   // float4 per row
  w.col4 = w.slice * L4;                             // first float4 column of the slice
  w.b = fast_div(w.u, a.div_H);
  w.hh = w.u - w.b * a.H;
  return w;
}

// The slice of every token's data row (g_t for V, the query half for K):
// loads issued (into v) by kd_stage_load, stored by kd_stage_store.
// Columns past the row read zero; indices past the data re-read an entry in
// range and are masked, so every load goes out at once.
constexpr int kKdStageMax = kKdDataBytes / 16 / kKdThreads;   // float4 per thread at most

template <int L4>
__device__ __forceinline__ void kd_stage_load(const ChunkArgs& a, const KdWho& w, float4 (&v)[kKdStageMax]) {
  const int T = a.T, tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kKdStageMax; ++j) {
    const int idx = tid + j * kKdThreads;
    const int t = min(idx / L4, T - 1), cc = idx & (L4 - 1);
    const int c = min(w.col4 + cc, w.width4 - 1);
    const float4* src = w.list == 0
        ? reinterpret_cast<const float4*>(a.g + ((int64_t)w.u * T + t) * a.dv)
        : reinterpret_cast<const float4*>(a.q + ((int64_t)(w.b * T + t) * a.H + w.hh) * a.dqk +
                                          (w.list - 1) * a.half);
    v[j] = src[c];
    const unsigned int mk = opaque_mask(w.col4 + cc < w.width4);
    v[j] = make_float4(__uint_as_float(__float_as_uint(v[j].x) & mk),
                       __uint_as_float(__float_as_uint(v[j].y) & mk),
                       __uint_as_float(__float_as_uint(v[j].z) & mk),
                       __uint_as_float(__float_as_uint(v[j].w) & mk));
  }
}

template <int L4>
__device__ __forceinline__ void kd_stage_store(int T, const float4 (&v)[kKdStageMax], float4* dat) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kKdStageMax; ++j) {
    const int idx = tid + j * kKdThreads;
    if (idx / L4 < T) dat[(idx / L4) * (L4 + 1) + (idx & (L4 - 1))] = v[j];
  }
}

// LDS scratch of the segment sums.
struct KdSeg {
  int* seg_beg;     // [cut + 1] segment starts, then the end
  int* seg_item;    // [cut] short index | first piece << 12 | first slot << 22
  int* short_seg;   // [cut] short segments in order
  int* items;       // [kKdMaxPieces] pieces of longer segments: segment << 5 | piece
  float4* part;     // [kKdMaxLong][L4] partial sums of pieces
  float* part_c;    // [kKdMaxLong] their coefficient sums
  int* long_seg;    // [kKdMaxLong] by slot: the segment whose first slot it is, else -1
  int* red;         // [4 * kKdWaves] block-scan scratch
};

// Checked builds: every entry [0, cut) in range, ordered by
// (hash_group(row, order_groups), row), and cut within the LDS lists.
template <int L4>
__device__ __forceinline__ void kd_check_entries(const ChunkArgs& a, const KdWho& who, const int* ent_row,
                                                 const int* ent_t, int cut, int order_groups) {
  const int tid = threadIdx.x;
  (void)a; (void)who; (void)ent_row; (void)ent_t; (void)cut; (void)order_groups; (void)tid;
#if FWPKM_DEVICE_CHECKS
  {
    const int rows = who.list == 0 ? a.n * a.n : a.n;
#pragma unroll
    for (int j = 0; j < kKdPer; ++j) {
      const int e = tid * kKdPer + j;
      if (e < cut) {
        device_check(a, ent_row[e] >= 0 && ent_row[e] < rows && ent_t[e] >= 0 && ent_t[e] < a.T, kChkEntry);
        if (e > 0) {
          const int r0 = ent_row[e - 1], r1 = ent_row[e];
          const int g0 = hash_group(r0, order_groups), g1 = hash_group(r1, order_groups);
          device_check(a, g0 < g1 || (g0 == g1 && r0 <= r1), kChkOrder);
        }
      }
    }
    if (tid == 0) device_check(a, cut <= kKdEntCap, kChkCapacity);
  }
#endif
}

// The sums of segments whose tables are built: segment s is entries
// [seg_beg[s], seg_beg[s + 1]), its fields in seg_item[s] (short index |
// first piece << 12 | first slot << 22); short segments listed in
// short_seg, pieces of longer ones in items (segment << 5 | piece), the
// first slot of each segment of more than kKdPiece pairs in long_seg (-1 on
// the rest).  Each row's mean gradient is applied to its slice of the table.
// Ends after a barrier-free phase: the caller synchronises before reusing
// the scratch.
template <int L4>
__device__ __forceinline__ void kd_segment_sums(const ChunkArgs& a, const KdWho& who, const float4* dat,
                                                const int* ent_row, const int* ent_t, const int* ent_w,
                                                const KdSeg& S, int nshort, int npieces, int nslots) {
  int* seg_beg = S.seg_beg;
  int* seg_item = S.seg_item;
  int* short_seg = S.short_seg;
  int* items = S.items;
  float4* part = S.part;
  float* part_c = S.part_c;
  int* long_seg = S.long_seg;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int c4 = lane & (L4 - 1), pg = lane / L4;
  const int width4 = who.width4, col4 = who.col4;
  const bool col_ok = col4 + c4 < width4;
  const float lr = a.lr;
  const bool idw_key = who.list != 0 && a.mode == 0;
  float* tbase = who.list == 0
      ? a.v + (int64_t)who.b * a.stride_v + (int64_t)who.hh * a.n * a.n * a.dv
      : (who.list == 1 ? a.k1 : a.k2) + (int64_t)who.b * a.stride_k + (int64_t)who.hh * a.n * a.half;
  const int rstride = who.list == 0 ? a.dv : a.half;

  {
    constexpr int PG = kWave / L4;
    if (tid == 0) device_check(a, nshort <= kKdEntCap && npieces <= kKdMaxPieces && nslots <= kKdMaxLong, kChkCapacity);
    const int npass = (nshort + PG - 1) / PG;

    // ---- short segments: pass i takes segments i*PG .. i*PG + PG - 1,
    // pair group g the g-th; lane g*L4 + j holds pair j of its segment.
    // Waves take passes wave, wave + W, ...; each lane fetches its own
    // segment's old row value ahead, KS passes per round (unrolled, so no
    // loop head between the prefetch and its use waits for the loads).
    constexpr int KS = 4;
    for (int j0 = 0; wave + j0 * kKdWaves < npass; j0 += KS) {
      float4 old[KS];
      int row[KS], len[KS], my_t[KS], my_w[KS];
#pragma unroll
      for (int r = 0; r < KS; ++r) {
        const int sidx = min(wave + (j0 + r) * kKdWaves, npass - 1) * PG + pg;
        const int si = short_seg[min(sidx, nshort - 1)];
        const int s0 = seg_beg[si];
        len[r] = sidx < nshort ? seg_beg[si + 1] - s0 : 0;
        row[r] = ent_row[s0];
        my_t[r] = ent_t[s0 + min(c4, max(len[r] - 1, 0))];
        my_w[r] = c4 < len[r] ? ent_w[s0 + c4] : 0;
        old[r] = reinterpret_cast<const float4*>(tbase + (int64_t)row[r] * rstride)[min(col4 + c4, width4 - 1)];
      }
#pragma unroll
      for (int r = 0; r < KS; ++r) {
        if (wave + (j0 + r) * kKdWaves >= npass) break;         // wave-uniform
        int steps = len[r];
        if constexpr (L4 <= 4) steps = max(steps, xor_lane<4>(steps));
        if constexpr (L4 <= 8) steps = max(steps, xor_lane<8>(steps));
        if constexpr (L4 <= 16) steps = max(steps, xor_lane<16>(steps));
        steps = __builtin_amdgcn_readfirstlane(max(steps, xor_lane<32>(steps)));
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float cs = 0.f;
        sum_steps<L4, 0>(steps, my_t[r], my_w[r], dat, c4, acc, cs);
        if (r == 0) {
          // every prefetched value is taken in before the round's first
          // store: a later wait for one of them would otherwise also wait
          // for the stores issued since (one counter covers both)
#pragma unroll
          for (int rr = 0; rr < KS; ++rr)
            asm volatile("" :: "v"(old[rr].x), "v"(old[rr].y), "v"(old[rr].z), "v"(old[rr].w));
        }
        if (len[r] > 0 && col_ok) {
          float4 x = old[r];
          const float inv = __builtin_amdgcn_rcpf((float)len[r]);
          if (idw_key) {
            acc.x = fmaf(-cs, x.x, acc.x); acc.y = fmaf(-cs, x.y, acc.y);
            acc.z = fmaf(-cs, x.z, acc.z); acc.w = fmaf(-cs, x.w, acc.w);
          }
          x.x -= lr * (acc.x * inv); x.y -= lr * (acc.y * inv);
          x.z -= lr * (acc.z * inv); x.w -= lr * (acc.w * inv);
          reinterpret_cast<float4*>(tbase + (int64_t)row[r] * rstride)[col4 + c4] = x;
        }
      }
    }

    // ---- pieces of longer segments, continuing the waves' turns: lane
    // g*L4 + j holds pair j*PG + g of the piece, pair groups are added by a
    // butterfly.  A one-piece segment is finished by lane group jj of its
    // round, whose prefetch register r holds its old row value.
    constexpr int KP = PG >= 16 ? 1 : kKdPrefetch;
    constexpr int R = KP * PG;
    const int w0 = (wave - npass % kKdWaves + kKdWaves) % kKdWaves;
    for (int j0 = 0; w0 + j0 * kKdWaves < npieces; j0 += R) {
      float4 old[KP];
#pragma unroll
      for (int r = 0; r < KP; ++r) {
        const int it = min(w0 + (j0 + r * PG + pg) * kKdWaves, npieces - 1);
        const int s0 = seg_beg[items[it] >> 5];
        old[r] = reinterpret_cast<const float4*>(tbase + (int64_t)ent_row[s0] * rstride)[min(col4 + c4, width4 - 1)];
      }
#pragma unroll
      for (int r = 0; r < KP; ++r) {
#pragma unroll
        for (int jj = 0; jj < PG; ++jj) {
          const int it = w0 + (j0 + r * PG + jj) * kKdWaves;
          if (it >= npieces) break;                              // wave-uniform
          const int packed = items[it];
          const int si = packed >> 5, q = packed & 31;
          const int s0 = seg_beg[si];
          const int len = __builtin_amdgcn_readfirstlane(seg_beg[si + 1] - s0);
          const int e0 = s0 + q * kKdPiece;
          const int np = min(kKdPiece, len - q * kKdPiece);
          const int pj = c4 * PG + pg;
          const int my_t = ent_t[e0 + min(pj, np - 1)];
          const int my_w = pj < np ? ent_w[e0 + pj] : 0;
          float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
          float cs = 0.f;
          sum_steps<L4, 0>((np + PG - 1) / PG, my_t, my_w, dat, c4, acc, cs);
          pair_group_sum<L4>(acc, cs);
          if (r == 0 && jj == 0) {
#pragma unroll
            for (int rr = 0; rr < KP; ++rr)
              asm volatile("" :: "v"(old[rr].x), "v"(old[rr].y), "v"(old[rr].z), "v"(old[rr].w));
          }
          if (len <= kKdPiece) {
            if (pg == jj && col_ok) {
              float4 x = old[r];
              const float inv = __builtin_amdgcn_rcpf((float)len);
              if (idw_key) {
                acc.x = fmaf(-cs, x.x, acc.x); acc.y = fmaf(-cs, x.y, acc.y);
                acc.z = fmaf(-cs, x.z, acc.z); acc.w = fmaf(-cs, x.w, acc.w);
              }
              x.x -= lr * (acc.x * inv); x.y -= lr * (acc.y * inv);
              x.z -= lr * (acc.z * inv); x.w -= lr * (acc.w * inv);
              reinterpret_cast<float4*>(tbase + (int64_t)ent_row[s0] * rstride)[col4 + c4] = x;
            }
          } else {
            const int slot = (seg_item[si] >> 22) + q;
            if (pg == 0) part[slot * L4 + c4] = acc;
            if (lane == 0) part_c[slot] = cs;
          }
        }
      }
    }
    __syncthreads();
    // ---- long segments: add the pieces in order and finish the row
    for (int slot0 = wave; slot0 < nslots; slot0 += kKdWaves) {
      const int si = long_seg[slot0];
      if (si < 0) continue;                                      // not a segment's first slot
      const int s0 = seg_beg[si];
      const int len = seg_beg[si + 1] - s0;
      const int pieces = (len + kKdPiece - 1) / kKdPiece;
      if (lane < L4 && col_ok) {
        float4* trow = reinterpret_cast<float4*>(tbase + (int64_t)ent_row[s0] * rstride) + col4 + c4;
        float4 x = *trow;
        float4 acc = part[slot0 * L4 + c4];
        float cs = part_c[slot0];
        for (int q = 1; q < pieces; ++q) {
          acc = f4_add(acc, part[(slot0 + q) * L4 + c4]);
          cs += part_c[slot0 + q];
        }
        const float inv = __builtin_amdgcn_rcpf((float)len);
        if (idw_key) {
          acc.x = fmaf(-cs, x.x, acc.x); acc.y = fmaf(-cs, x.y, acc.y);
          acc.z = fmaf(-cs, x.z, acc.z); acc.w = fmaf(-cs, x.w, acc.w);
        }
        x.x -= lr * (acc.x * inv); x.y -= lr * (acc.y * inv);
        x.z -= lr * (acc.z * inv); x.w -= lr * (acc.w * inv);
        *trow = x;
      }
    }
  }
}


// The segments (runs of one row) of the entries [0, cut), in LDS: rows
// ent_row, tokens ent_t, weights ent_w (float bits), ordered by
// (hash_group(row, order_groups), row) -- by row alone with one group --
// so every row's entries are one run: their tables, then their sums.
// cut <= kKdEntCap.  Ends like kd_segment_sums.
template <int L4>
__device__ __forceinline__ void kd_sum_segments(const ChunkArgs& a, const KdWho& who,
                                                const float4* dat, const int* ent_row,
                                                const int* ent_t, const int* ent_w, int cut,
                                                const KdSeg& S, int order_groups) {
  int* seg_beg = S.seg_beg;
  int* seg_item = S.seg_item;
  int* short_seg = S.short_seg;
  int* items = S.items;
  int* long_seg = S.long_seg;
  int* red = S.red;
  const int tid = threadIdx.x;
  kd_check_entries<L4>(a, who, ent_row, ent_t, cut, order_groups);
  // entries tid * kKdPer + j: contiguous per thread, so segment starts
  // come out in order from one scan
  bool hd[kKdPer];
  int nh = 0;
#pragma unroll
  for (int j = 0; j < kKdPer; ++j) {
    const int e = tid * kKdPer + j;
    hd[j] = e < cut && (e == 0 || ent_row[e] != ent_row[e - 1]);
    nh += hd[j];
  }
  int nseg;
  int sp = kd_block_scan(nh, red, &nseg);
#pragma unroll
  for (int j = 0; j < kKdPer; ++j)
    if (hd[j]) seg_beg[sp++] = tid * kKdPer + j;
  if (tid == 0) seg_beg[nseg] = cut;
  __syncthreads();
  // ---- work.  A segment of at most L4 pairs is short: kWave / L4 of them
  // share one pass of a wave, one per pair group.  A longer segment is cut
  // into kKdPiece-pair pieces, each summed by a whole wave; the pieces of a
  // segment longer than kKdPiece meet in `part`.
  {
    int sh[kKdPer], pcs[kKdPer], slt[kKdPer], tot = 0;
#pragma unroll
    for (int j = 0; j < kKdPer; ++j) {
      const int si = tid * kKdPer + j;
      const int len = si < nseg ? seg_beg[si + 1] - seg_beg[si] : 0;
      sh[j] = si < nseg && len <= L4 ? 1 : 0;
      pcs[j] = len > L4 ? (len + kKdPiece - 1) / kKdPiece : 0;
      slt[j] = len > kKdPiece ? pcs[j] : 0;
      tot += sh[j] | (pcs[j] << 12) | (slt[j] << 22);
    }
    int total;
    int pre = kd_block_scan(tot, red + 2 * kKdWaves, &total);
#pragma unroll
    for (int j = 0; j < kKdPer; ++j) {
      const int si = tid * kKdPer + j;
      if (si < nseg) {
        seg_item[si] = pre;          // short index | first piece << 12 | first slot << 22
        if (sh[j]) short_seg[pre & 0xfff] = si;
        for (int q = 0; q < pcs[j]; ++q) items[((pre >> 12) & 0x3ff) + q] = (si << 5) | q;
        for (int q = 0; q < slt[j]; ++q) long_seg[(pre >> 22) + q] = q == 0 ? si : -1;
      }
      pre += sh[j] | (pcs[j] << 12) | (slt[j] << 22);
    }
    __syncthreads();
    const int nshort = total & 0xfff;
    const int npieces = (total >> 12) & 0x3ff;
    const int nslots = total >> 22;
    kd_segment_sums<L4>(a, who, dat, ent_row, ent_t, ent_w, S, nshort, npieces, nslots);
  }
}

}  // namespace

// Large chunks: entries grouped by the grouping kernel (kc_sort).
template <int SW>
__global__ __launch_bounds__(kKdThreads) void kd_update(ChunkArgs a) {
  constexpr int L4 = SW / 4;                 // float4 columns of a slice
  extern __shared__ float4 kd_lds4[];
  char* lds = reinterpret_cast<char*>(kd_lds4);
  const KdLds LL = kd_lds_layout(a.T, SW);
  float4* dat = reinterpret_cast<float4*>(lds + LL.dat);
  int* ent_t = reinterpret_cast<int*>(lds + LL.ent_t);
  int* ent_w = reinterpret_cast<int*>(lds + LL.ent_w);        // float bits
  int* ent_row = reinterpret_cast<int*>(lds + LL.ent_row);
  KdSeg S;
  S.seg_beg = reinterpret_cast<int*>(lds + LL.seg_beg);
  S.seg_item = reinterpret_cast<int*>(lds + LL.seg_item);
  S.short_seg = reinterpret_cast<int*>(lds + LL.short_seg);
  S.items = reinterpret_cast<int*>(lds + LL.items);
  S.part = reinterpret_cast<float4*>(lds + LL.part);
  S.part_c = reinterpret_cast<float*>(lds + LL.part_c);
  S.long_seg = reinterpret_cast<int*>(lds + LL.long_seg);
  S.red = reinterpret_cast<int*>(lds + LL.red);               // [4][kKdWaves]
  int* red = S.red;

  // every launch argument the prologue needs, fetched in one batch with one
  // wait (see kd_write)
  asm volatile("" :: "s"(a.T), "s"(a.U), "s"(a.kd_pu), "s"(a.kd_div_pu.m), "s"(a.kd_div_pu.l), "s"(a.kd_sv),
               "s"(a.kd_gv), "s"(a.kd_div_gv.m), "s"(a.kd_div_gv.l), "s"(a.kd_sk), "s"(a.kd_gk),
               "s"(a.kd_div_kl.m), "s"(a.kd_div_kl.l), "s"(a.kd_div_gk.m), "s"(a.kd_div_gk.l), "s"(a.dv),
               "s"(a.half), "s"(a.div_H.m), "s"(a.div_H.l), "s"(a.H), "s"(a.P), "s"(a.regions), "s"(a.kinds),
               "s"(a.ent_row), "s"(a.ent_tw));
  const KdWho who = kd_who(a, L4);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int64_t lbase = ((int64_t)who.list * a.U + who.u) * a.P;

  // ---- this group's run of entries: regions [r0, r0 + RG).  Every wave
  // reads the (at most 64) region records itself, so the entry loads need
  // no barrier.
  const int RG = a.regions / who.ngrp;                    // groups are runs of regions
  const int r0 = who.grp * RG;
  int4 kd = make_int4(0, 0, 0, 0);
  if (lane < RG) kd = a.kinds[((int64_t)who.list * a.U + who.u) * a.regions + r0 + lane];
  const int e_count = wave_sum(lane < RG ? kd.w : 0);
  const int e_first = readlane_i(kd.z, 0);               // the first region's offset
  if (tid == 0) device_check(a, e_first >= 0 && e_count >= 0 && e_first + e_count <= a.P, kChkCapacity);
  if (e_count == 0) return;                               // block-uniform: nothing to write
  const int* erow = a.ent_row + lbase + e_first;
  const int2* etw = a.ent_tw + lbase + e_first;

  // ---- a batch's entries and the row after it (if any) into LDS
  int rv[kKdPer];
  int2 tw[kKdPer];
  int after = 0;
  auto load_batch = [&](int done, int n, bool last) {
#pragma unroll
    for (int j = 0; j < kKdPer; ++j) {
      const int e = min(tid + j * kKdThreads, n - 1);
      rv[j] = erow[done + e];
      tw[j] = etw[done + e];
    }
    after = erow[done + (last ? n - 1 : n)];
  };
  auto store_batch = [&](int n, bool last) {
#pragma unroll
    for (int j = 0; j < kKdPer; ++j) {
      const int e = tid + j * kKdThreads;
      if (e < n) {
        ent_row[e] = rv[j];
        ent_t[e] = tw[j].x;
        ent_w[e] = tw[j].y;
      }
    }
    if (tid == 0) ent_row[n] = last ? -1 : after;
  };
  {
    // the first batch's entries go out first and the data slice right
    // behind them: loads complete in order, so the entries are stored while
    // the slice is still on its way
    const int n = min(kKdEntCap, e_count);
    load_batch(0, n, n == e_count);
    float4 v[kKdStageMax];
    kd_stage_load<L4>(a, who, v);
    store_batch(n, n == e_count);
    kd_stage_store<L4>(a.T, v, dat);
  }

  for (int done = 0; done < e_count;) {             // block-uniform
    const int n = min(kKdEntCap, e_count - done);
    const bool last = done + n == e_count;
    if (done > 0) {
      load_batch(done, n, last);
      store_batch(n, last);
    }
    __syncthreads();
    // ---- unless this is the last batch, it ends at its last segment head
    // (a segment is at most one pair per token, shorter than a batch, so one
    // exists past entry 0)
    int cut = n;
    if (!last) {
      int hmax = 0;
#pragma unroll
      for (int j = 0; j < kKdPer; ++j) {
        const int e = tid + j * kKdThreads + 1;          // heads in (0, n]
        if (e <= n && ent_row[e] != ent_row[e - 1]) hmax = max(hmax, e);
      }
      hmax = max(hmax, xor_lane<32>(hmax));
      hmax = max(hmax, xor_lane<16>(hmax));
      hmax = max(hmax, xor_lane<8>(hmax));
      hmax = max(hmax, xor_lane<4>(hmax));
      hmax = max(hmax, xor_lane<2>(hmax));
      hmax = max(hmax, xor_lane<1>(hmax));
      if (lane == 0) red[kKdWaves + wave] = hmax;
      __syncthreads();
      cut = 0;
#pragma unroll
      for (int w = 0; w < kKdWaves; ++w) cut = max(cut, red[kKdWaves + w]);
    }
    kd_sum_segments<L4>(a, who, dat, ent_row, ent_t, ent_w, cut, S, a.regions);
    done += cut;
    __syncthreads();                 // the staged entries are reused
  }
}

// ints of the fused kernel's digit counters, later segment starts and items
constexpr int kKwCntInts = (kKdWaves * 256 > 2 * kKdEntCap + 1 ? kKdWaves * 256 : 2 * kKdEntCap + 1) + 64;

// LDS layout (byte offsets) of the fused kernel: chunks of T tokens, slices
// of SW floats, at most kKdEntCap pairs per unit.
struct KwLds {
  int dat, key0, idx0, key1, idx1, wl, cnt, items, part, part_c, long_seg, red, dbeg, ditem, dshort, total;
};
__host__ __device__ constexpr KwLds kw_lds_layout(int T, int SW) {
  KwLds L{};
  int o = 0;
  L.key0 = o;   o = kd_align(o + kKdEntCap * 4);                  // sort ping: rows, pair indices
  L.idx0 = o;   o = kd_align(o + kKdEntCap * 4);
  L.key1 = o;   o = kd_align(o + kKdEntCap * 4);                  // pong (later tokens, weights)
  L.idx1 = o;   o = kd_align(o + kKdEntCap * 4);
  L.wl = o;     o = kd_align(o + kKdEntCap * 4);                  // weight of each pair (later short segments)
  L.cnt = o;    o = kd_align(o + kKwCntInts * 4);                 // digit counters (later segment starts, items)
  L.items = o;  o = kd_align(o + kKdMaxPieces * 4);
  L.part = o;   o = kd_align(o + kKdMaxLong * (SW / 4) * 16);
  L.part_c = o; o = kd_align(o + kKdMaxLong * 4);
  L.long_seg = o; o = kd_align(o + kKdMaxLong * 4);
  L.red = o;    o = kd_align(o + 4 * kKdWaves * 4);
  L.dbeg = o;   o = kd_align(o + (256 + 1) * 4);                  // segment tables when one digit is one row
  L.ditem = o;  o = kd_align(o + 256 * 4);
  L.dshort = o; o = kd_align(o + 256 * 4);
  L.dat = o;    o = kd_align(o + T * (SW / 4 + 1) * 16);          // last: the one T-dependent part
  L.total = o;
  return L;
}
static_assert(2 * kKdEntCap + 1 <= kKwCntInts, "segment starts and items fit the counters' space");

// Chunks of at most kKdEntCap pairs per unit: grouping fused in.
template <int SW>
__global__ __launch_bounds__(kKdThreads) void kd_write(ChunkArgs a) {
  constexpr int L4 = SW / 4;
  constexpr int kTiles = kKdEntCap / kWave / kKdWaves;   // list tiles per wave at most (2)
  extern __shared__ float4 kd_lds4[];
  char* lds = reinterpret_cast<char*>(kd_lds4);
  const KwLds LL = kw_lds_layout(a.T, SW);
  float4* dat = reinterpret_cast<float4*>(lds + LL.dat);
  int* key0 = reinterpret_cast<int*>(lds + LL.key0);
  int* idx0 = reinterpret_cast<int*>(lds + LL.idx0);
  int* key1 = reinterpret_cast<int*>(lds + LL.key1);
  int* idx1 = reinterpret_cast<int*>(lds + LL.idx1);
  int* wl = reinterpret_cast<int*>(lds + LL.wl);
  int* cnt = reinterpret_cast<int*>(lds + LL.cnt);
  int* red = reinterpret_cast<int*>(lds + LL.red);

  // every launch argument the prologue needs, as scalar operands of an empty
  // statement: they are fetched in one batch with one wait.  Left to itself
  // the compiler fetches them in dependent rounds, and with 16 waves taking
  // turns on the compute unit's scalar unit the last wave then issued its
  // first loads ~0.5 us after the first.
  asm volatile("" :: "s"(a.T), "s"(a.U), "s"(a.kd_pu), "s"(a.kd_div_pu.m), "s"(a.kd_div_pu.l), "s"(a.kd_sv),
               "s"(a.kd_gv), "s"(a.kd_div_gv.m), "s"(a.kd_div_gv.l), "s"(a.kd_sk), "s"(a.kd_gk),
               "s"(a.kd_div_kl.m), "s"(a.kd_div_kl.l), "s"(a.kd_div_gk.m), "s"(a.kd_div_gk.l), "s"(a.dv),
               "s"(a.half), "s"(a.div_H.m), "s"(a.div_H.l), "s"(a.H), "s"(a.P), "s"(a.keys), "s"(a.sel_w),
               "s"(a.coef), "s"(a.n));
  const KdWho who = kd_who(a, L4);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int P = a.P;
  const int64_t lbase = ((int64_t)who.list * a.U + who.u) * P;
  const int* keys = a.keys + lbase;
  const float* wsrc = who.list == 0 ? a.sel_w + (int64_t)who.u * P
                                    : a.coef + (int64_t)(who.list - 1) * a.U * P + (int64_t)who.u * P;
  const int invalid = who.list == 0 ? a.n * a.n : a.n;

  // ---- the list's rows and weights.  Wave w owns list tiles
  // [w*tpw, (w+1)*tpw), so kept entries come out in pair order; indices past
  // the list re-read entry 0 and are masked.
  const int tiles = (int)(((unsigned)P + kWave - 1) / kWave);
  const int tpw = (int)(((unsigned)tiles + kKdWaves - 1) / kKdWaves);   // <= kTiles
  int kr[kTiles];
  float wr[kTiles];
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    const int i = (wave * tpw + j) * kWave + lane;
    const int ic = j < tpw && i < P ? i : 0;
    kr[j] = keys[ic];
    wr[j] = wsrc[ic];
  }
  reinterpret_cast<int4*>(cnt + wave * 256)[lane] = make_int4(0, 0, 0, 0);   // this wave's digit counters
  // radix passes the rows need (8-bit digits)
  const int passes = max(1, (bit_length(invalid - 1) + 7) / 8);
  // rows of up to 16 bits (two passes) may be renamed to their rank among
  // the group's distinct rows: a bitmap of the rows present, in the segment
  // sums' scratch (free until then)
  static_assert(kKdMaxLong * 16 * 16 >= 2 * 2048 * 4, "bitmap and scan fit the sums' scratch at SW = 64");
  static_assert(kKdThreads * 2 == 2048, "two bitmap words per thread");
  const bool try_rename = SW == 64 && passes == 2;             // block-uniform
  unsigned int* bm = reinterpret_cast<unsigned int*>(lds + LL.part);   // [2048] words
  int* wpre = reinterpret_cast<int*>(lds + LL.part) + 2048;            // [2048]
  if (try_rename) {
    bm[2 * tid] = 0u;
    bm[2 * tid + 1] = 0u;
  }
  int* items = reinterpret_cast<int*>(lds + LL.items);
  int* long_seg = reinterpret_cast<int*>(lds + LL.long_seg);
  int* dbeg = reinterpret_cast<int*>(lds + LL.dbeg);
  int* ditem = reinterpret_cast<int*>(lds + LL.ditem);
  int* dshort = reinterpret_cast<int*>(lds + LL.dshort);

  // ---- row masks.  At most 256 tokens, and rows that are (or are renamed
  // to) at most 256 ranks: each rank's tokens form a 256-bit mask, set by
  // LDS atomic ORs (the result does not depend on their order).  Within a
  // list a token touches a row at most once, so a rank's entries in token
  // order are exactly its entries in pair order, and an entry's place in
  // the grouped list is the entries of the ranks below plus the tokens of
  // its own rank below it (popcounts).  This gives the stable sort's output
  // without a compaction, digit ballots or a scatter pass.
  static_assert(256 * 8 * 2 <= kKwCntInts, "row masks and their starts fit the counters' space");
  constexpr bool kMaskT = SW == 64;                   // T <= 256: eight mask words per rank
  int D = 0;
  if (kMaskT && passes <= 2) {
    lds_barrier();                                    // counters and bitmap cleared; the rows' loads stay in flight
    if (try_rename) {
#pragma unroll
      for (int j = 0; j < kTiles; ++j) {
        const int i = (wave * tpw + j) * kWave + lane;
        const bool mine = j < tpw && i < P && kr[j] != invalid && hash_group(kr[j], who.ngrp) == who.grp;
        if (mine) atomicOr(&bm[(unsigned)kr[j] >> 5], 1u << (kr[j] & 31));
      }
      lds_barrier();
      const unsigned int w0 = bm[2 * tid], w1 = bm[2 * tid + 1];
      const int pre = kd_block_scan<true>(__popc(w0) + __popc(w1), red, &D);
      if (D == 0) return;                             // block-uniform: nothing to write
      wpre[2 * tid] = pre;
      wpre[2 * tid + 1] = pre + __popc(w0);
      lds_barrier();
    }
  }
  if (kMaskT && (passes == 1 || (try_rename && D <= 256))) {   // block-uniform
    unsigned int* rmask = reinterpret_cast<unsigned int*>(cnt);   // [256][8] tokens of each rank
    int* rstart = cnt + 256 * 8;                                  // [256][8] first place of each mask word
    float4 v[kKdStageMax];
    kd_stage_load<L4>(a, who, v);                     // the data slice travels while the rows are grouped
    int rk[kTiles], tk[kTiles];
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      const int i = (wave * tpw + j) * kWave + lane;
      const bool mine = j < tpw && i < P && kr[j] != invalid && hash_group(kr[j], who.ngrp) == who.grp;
      rk[j] = -1;
      tk[j] = 0;
      if (mine) {
        const int r = kr[j];
        rk[j] = try_rename ? wpre[r >> 5] + __popc(bm[r >> 5] & ((1u << (r & 31)) - 1u)) : r;
        tk[j] = token_of(i, a.k);
        atomicOr(&rmask[rk[j] * 8 + (tk[j] >> 5)], 1u << (tk[j] & 31));
      }
    }
    lds_barrier();
    // entries per rank, their starts (a scan over ranks by waves 0-3) and
    // the segment tables: every rank with entries is one segment, its
    // fields short (at most L4 pairs), pieces of kKdPiece pairs, slots of
    // segments longer than one piece
    uint4 m0 = make_uint4(0u, 0u, 0u, 0u), m1 = m0;
    int run = 0, dbase = 0, nz = 0, pk = 0, inz = 0, ipk = 0, pcs = 0, slt = 0;
    if (tid < 256) {                                  // whole waves 0-3
      m0 = reinterpret_cast<const uint4*>(rmask)[2 * tid];
      m1 = reinterpret_cast<const uint4*>(rmask)[2 * tid + 1];
      run = __popc(m0.x) + __popc(m0.y) + __popc(m0.z) + __popc(m0.w) +
            __popc(m1.x) + __popc(m1.y) + __popc(m1.z) + __popc(m1.w);
      const int incl = wave_inclusive_scan(run);
      dbase = incl - run;
      nz = run > 0 ? 1 : 0;
      pcs = run > L4 ? (run + kKdPiece - 1) / kKdPiece : 0;
      slt = run > kKdPiece ? pcs : 0;
      pk = nz ? ((run <= L4 ? 1 : 0) | (pcs << 12) | (slt << 22)) : 0;
      inz = wave_inclusive_scan(nz);
      ipk = wave_inclusive_scan(pk);
      if (lane == kWave - 1) {
        red[wave] = incl;
        red[kKdWaves + wave] = inz;
        red[2 * kKdWaves + wave] = ipk;
      }
    }
    lds_barrier();
    if (tid < 256) {
      int bz = 0, bp = 0;
      for (int w = 0; w < wave; ++w) {
        dbase += red[w];
        bz += red[kKdWaves + w];
        bp += red[2 * kKdWaves + w];
      }
      int4 s0, s1;
      int s = dbase;
      s0.x = s; s += __popc(m0.x);
      s0.y = s; s += __popc(m0.y);
      s0.z = s; s += __popc(m0.z);
      s0.w = s; s += __popc(m0.w);
      s1.x = s; s += __popc(m1.x);
      s1.y = s; s += __popc(m1.y);
      s1.z = s; s += __popc(m1.z);
      s1.w = s;
      reinterpret_cast<int4*>(rstart)[2 * tid] = s0;
      reinterpret_cast<int4*>(rstart)[2 * tid + 1] = s1;
      const int sgi = bz + inz - nz;                  // segment number of this rank
      const int pp = bp + ipk - pk;                   // fields of the segments before it
      if (nz) {
        dbeg[sgi] = dbase;
        ditem[sgi] = pp;
        if (run <= L4) dshort[pp & 0xfff] = sgi;
        for (int q = 0; q < pcs; ++q) items[((pp >> 12) & 0x3ff) + q] = (sgi << 5) | q;
        for (int q = 0; q < slt; ++q) long_seg[(pp >> 22) + q] = q == 0 ? sgi : -1;
      }
      if (tid == 255) {
        dbeg[bz + inz] = dbase + run;
        red[3 * kKdWaves] = bp + ipk;                 // totals of the fields
        red[3 * kKdWaves + 1] = dbase + run;          // entries
      }
    }
    lds_barrier();
    const int M = red[3 * kKdWaves + 1];
    const int tot = red[3 * kKdWaves];
    if (M == 0) {                                     // block-uniform: nothing to write
      kd_stage_store<L4>(a.T, v, dat);                // (the slice's loads land before the exit)
      return;
    }
    // each entry to its place: rows, tokens and weights grouped by rank
    int* ks = key0;
    int* ent_t = key1;
    int* ent_w = idx1;
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      if (rk[j] >= 0) {
        const int wi = rk[j] * 8 + (tk[j] >> 5);
        const int pos = rstart[wi] + __popc(rmask[wi] & ((1u << (tk[j] & 31)) - 1u));
        ks[pos] = kr[j];
        ent_t[pos] = tk[j];
        ent_w[pos] = __float_as_int(wr[j]);
      }
    }
    kd_stage_store<L4>(a.T, v, dat);
    __syncthreads();
    KdSeg S;
    S.items = items;
    S.part = reinterpret_cast<float4*>(lds + LL.part);
    S.part_c = reinterpret_cast<float*>(lds + LL.part_c);
    S.long_seg = long_seg;
    S.red = red;
    S.seg_beg = dbeg;
    S.seg_item = ditem;
    S.short_seg = dshort;
    kd_check_entries<L4>(a, who, ks, ent_t, M, 1);
    kd_segment_sums<L4>(a, who, dat, ks, ent_t, ent_w, S, tot & 0xfff, (tot >> 12) & 0x3ff, tot >> 22);
    return;
  }
  // ---- otherwise a stable LSD radix sort.  Keep this group's rows, in
  // pair order
  int kept = 0;
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    const int i = (wave * tpw + j) * kWave + lane;
    const bool in = j < tpw && i < P;
    if (in) wl[i] = __float_as_int(wr[j]);
    const bool mine = in && kr[j] != invalid && hash_group(kr[j], who.ngrp) == who.grp;
    kept += __popcll(__ballot(mine));
  }
  if (lane == 0) red[wave] = kept;
  lds_barrier();
  int base = 0, M = 0;
#pragma unroll
  for (int w = 0; w < kKdWaves; ++w) {
    const int t = red[w];
    base += w < wave ? t : 0;
    M += t;
  }
  if (M == 0) return;                                 // block-uniform: nothing to write
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    const int i = (wave * tpw + j) * kWave + lane;
    const bool in = j < tpw && i < P;
    const bool mine = in && kr[j] != invalid && hash_group(kr[j], who.ngrp) == who.grp;
    const unsigned long long m = __ballot(mine);
    if (mine) {
      const int pos = base + __popcll(m & lanes_below());
      key0[pos] = kr[j];
      idx0[pos] = i;
    }
    base += __popcll(m);
  }
  lds_barrier();

  // ---- stable LSD radix sort of the M kept (row, pair) by row: 8-bit
  // digits, as many passes as the largest row needs.  Wave w owns entry
  // tiles [t_lo, t_hi) and its own digit counters; the scatter base of a
  // (digit, wave) is an exclusive scan in digit-major order.
  const int vtiles = (M + kWave - 1) / kWave;
  const int vtpw = (vtiles + kKdWaves - 1) / kKdWaves;
  const int t_lo = wave * vtpw, t_hi = min(vtiles, t_lo + vtpw);
  int* mycnt = cnt + wave * 256;
  int *ks = key0, *is = idx0, *kd = key1, *id = idx1;
  // one pass whose digit is the row: the segments are the digits present,
  // and the last pass's scan builds their tables
  const bool direct = passes == 1;
  // the data slice, stored to LDS only after the sort: its loads travel
  // while the radix passes run (the grouping's barriers order LDS alone).
  // Issued beside the rows, they queued ahead of the later waves' row loads
  // in the compute unit's load path and held the compaction back ~1 us;
  // issued before the compaction, the waves stalled issuing them.
  float4 v[kKdStageMax];
  kd_stage_load<L4>(a, who, v);
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * 8;
    // each tile's lanes with equal digits (ballots), counted once by the
    // lowest of them into this wave's own counters (no other wave writes
    // them, and a wave's LDS operations complete in order, so no atomics);
    // keys, digits and peer masks stay in registers for the scatter
    int tk[kTiles], td[kTiles];
    unsigned long long tp[kTiles];
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      if (t_lo + j >= t_hi) break;                     // wave-uniform: ballots run on the shared scalar unit
      const int i = (t_lo + j) * kWave + lane;
      const bool valid = i < M;
      tk[j] = valid ? ks[i] : 0;
      td[j] = ((unsigned)tk[j] >> shift) & 255;
      tp[j] = digit_peers(td[j], valid);
      if (valid && (tp[j] & lanes_below()) == 0ull) mycnt[td[j]] += __popcll(tp[j]);
    }
    lds_barrier();
    // scatter bases in digit-major, wave-minor order, digit-parallel: thread
    // d < 256 (waves 0-3) runs over the waves' counters of digit d, then the
    // digits' totals are scanned across those four waves.  When the digit is
    // the row (last pass of the direct path), the same scan numbers the
    // digits present (the segments) and sums their fields: short (at most
    // L4 pairs), pieces of kKdPiece pairs, slots of segments longer than one
    // piece.
    const bool tables = direct && pass == passes - 1;   // block-uniform
    int pre[kKdWaves];
    int dbase = 0, run = 0, nz = 0, pk = 0, inz = 0, ipk = 0, pcs = 0, slt = 0;
    if (tid < 256) {                                     // whole waves 0-3
#pragma unroll
      for (int w = 0; w < kKdWaves; ++w) {
        pre[w] = run;
        run += cnt[w * 256 + tid];
      }
      const int incl = wave_inclusive_scan(run);
      if (lane == kWave - 1) red[wave] = incl;
      dbase = incl - run;
      if (tables) {
        nz = run > 0 ? 1 : 0;
        pcs = run > L4 ? (run + kKdPiece - 1) / kKdPiece : 0;
        slt = run > kKdPiece ? pcs : 0;
        pk = nz ? ((run <= L4 ? 1 : 0) | (pcs << 12) | (slt << 22)) : 0;
        inz = wave_inclusive_scan(nz);
        ipk = wave_inclusive_scan(pk);
        if (lane == kWave - 1) {
          red[kKdWaves + wave] = inz;
          red[2 * kKdWaves + wave] = ipk;
        }
      }
    }
    lds_barrier();
    if (tid < 256) {
      int bz = 0, bp = 0;
      for (int w = 0; w < wave; ++w) {
        dbase += red[w];
        if (tables) {
          bz += red[kKdWaves + w];
          bp += red[2 * kKdWaves + w];
        }
      }
#pragma unroll
      for (int w = 0; w < kKdWaves; ++w) cnt[w * 256 + tid] = dbase + pre[w];
      if (tables) {
        const int sgi = bz + inz - nz;                 // segment number of this digit
        const int pp = bp + ipk - pk;                  // fields of the segments before it
        if (nz) {
          dbeg[sgi] = dbase;
          ditem[sgi] = pp;
          if (run <= L4) dshort[pp & 0xfff] = sgi;
          for (int q = 0; q < pcs; ++q) items[((pp >> 12) & 0x3ff) + q] = (sgi << 5) | q;
          for (int q = 0; q < slt; ++q) long_seg[(pp >> 22) + q] = q == 0 ? sgi : -1;
        }
        if (tid == 255) {
          dbeg[bz + inz] = M;
          red[3 * kKdWaves] = bp + ipk;                // totals of the fields
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      if (t_lo + j >= t_hi) break;                     // wave-uniform
      const int i = (t_lo + j) * kWave + lane;
      const bool valid = i < M;
      const unsigned long long lower = tp[j] & lanes_below();
      const int b0 = valid ? mycnt[td[j]] : 0;
      if (valid) {
        const int dst = b0 + __popcll(lower);
        kd[dst] = tk[j];
        id[dst] = is[i];
      }
      if (valid && lower == 0ull) mycnt[td[j]] = b0 + __popcll(tp[j]);
    }
    for (int i = lane; i < 256; i += kWave) mycnt[i] = 0;   // for the next pass
    lds_barrier();
    int* t;
    t = ks; ks = kd; kd = t;
    t = is; is = id; id = t;
  }
  // ---- the data slice into LDS; sorted entries: rows ks, tokens and
  // weights into the free buffers
  kd_stage_store<L4>(a.T, v, dat);
  int* ent_t = kd;
  int* ent_w = id;
  for (int i = tid; i < M; i += kKdThreads) {
    const int p = is[i];
    ent_t[i] = token_of(p, a.k);
    ent_w[i] = wl[p];
  }
  __syncthreads();
  KdSeg S;
  S.items = items;
  S.part = reinterpret_cast<float4*>(lds + LL.part);
  S.part_c = reinterpret_cast<float*>(lds + LL.part_c);
  S.long_seg = long_seg;
  S.red = red;
  if (direct) {
    S.seg_beg = dbeg;
    S.seg_item = ditem;
    S.short_seg = dshort;
    const int tot = red[3 * kKdWaves];
    kd_check_entries<L4>(a, who, ks, ent_t, M, 1);
    kd_segment_sums<L4>(a, who, dat, ks, ent_t, ent_w, S, tot & 0xfff, (tot >> 12) & 0x3ff, tot >> 22);
  } else {
    S.seg_beg = cnt;
    S.seg_item = cnt + kKdEntCap + 1;
    S.short_seg = wl;
    kd_sum_segments<L4>(a, who, dat, ks, ent_t, ent_w, M, S, 1);
  }
}

namespace {

// Column-slice width: the widest whose data for every token fits kKdDataBytes.
int kd_slice_width(int T) {
  return T * 64 * 4 <= kKdDataBytes ? 64 : (T * 32 * 4 <= kKdDataBytes ? 32 : 16);
}

template <int SW>
hipError_t launch_kd_as(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const int64_t per_unit = a.kd_pu;
  const dim3 grid((unsigned)(per_unit * a.U));
  if (kd_fuses_grouping(a)) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&kd_write<SW>), hipFuncAttributeMaxDynamicSharedMemorySize,
        kw_lds_layout(kKdDataBytes / (SW * 4), SW).total);
    if (attr != hipSuccess) return attr;
    return fw_launch(kd_write<SW>, grid, dim3(kKdThreads), (uint32_t)kw_lds_layout(a.T, SW).total, s, tm, a);
  }
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&kd_update<SW>), hipFuncAttributeMaxDynamicSharedMemorySize,
      kd_lds_layout(kKdDataBytes / (SW * 4), SW).total);
  if (attr != hipSuccess) return attr;
  return fw_launch(kd_update<SW>, grid, dim3(kKdThreads), (uint32_t)kd_lds_layout(a.T, SW).total, s, tm, a);
}

}  // namespace

bool kd_fuses_grouping(const ChunkArgs& a) { return a.P <= kKdEntCap; }

hipError_t launch_kd(const ChunkArgs& args, hipStream_t s, const LaunchTiming* tm) {
  ChunkArgs a = with_divisors(args);
  const int sw = kd_slice_width(a.T);
  a.kd_sv = (a.dv + sw - 1) / sw;
  a.kd_sk = (a.half + sw - 1) / sw;
  int gv = 1, gk = 1;
  if (kd_fuses_grouping(a)) {
    // hash groups per (list, unit): each workgroup sorts its group's entries
    // and sums them, so its work goes as entries x (radix passes + 1).  A
    // value list holds P entries over n^2 rows; a sub-key list about P/2 (a
    // token's candidates sharing a sub-key row are merged) over n rows.  The
    // counts (gv, gk) even out the two kinds of workgroup within one
    // workgroup per compute unit in all.
    auto passes = [](int64_t rows) { int b = 0; while (b < 40 && ((rows - 1) >> b) != 0) ++b; return (b + 7) / 8; };
    const double cost_v = (double)a.P * (passes((int64_t)a.n * a.n) + 1);
    const double cost_k = 0.5 * a.P * (passes(a.n) + 1);
    const int64_t most = std::max<int64_t>(256, (int64_t)a.U * (a.kd_sv + 2 * a.kd_sk));
    double best = 1e300;
    for (int v = 1; v <= 64; ++v)
      for (int q = 1; q <= 64; ++q) {
        if ((int64_t)a.U * (a.kd_sv * v + 2 * a.kd_sk * q) > most) break;
        const double c = std::max(cost_v / v, cost_k / q);
        if (c < best * (1.0 - 1e-9)) { best = c; gv = v; gk = q; }
      }
  } else {
    // unfused, a group is a run of the grouping kernel's regions (a power of
    // two of them): about one workgroup per compute unit in all, and about
    // two batches of entries per group at most (P / groups <= 2 kKdEntCap on
    // average), so that a list with many distinct rows does not leave half
    // the chip idle behind a few long workgroups
    const int combos = a.kd_sv + 2 * a.kd_sk;
    int sg = 1;
    while (sg * 2 <= a.regions && (int64_t)a.U * combos * sg * 2 <= 256) sg *= 2;
    while (sg * 2 <= a.regions && (int64_t)sg * 2 * kKdEntCap < a.P) sg *= 2;
    gv = gk = sg;
  }
  a.kd_gv = gv;
  a.kd_gk = gk;
  a.kd_pu = a.kd_sv * gv + 2 * a.kd_sk * gk;
  a.kd_div_pu = make_fastdiv(a.kd_pu);
  a.kd_div_gv = make_fastdiv(gv);
  a.kd_div_gk = make_fastdiv(gk);
  a.kd_div_kl = make_fastdiv(a.kd_sk * gk);
  if (sw == 64) return launch_kd_as<64>(a, s, tm);
  if (sw == 32) return launch_kd_as<32>(a, s, tm);
  return launch_kd_as<16>(a, s, tm);
}

}  // namespace fwpkm
