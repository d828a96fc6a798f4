// KC: deterministic grouping of the chunk's (row, pair) lists.
//
// One workgroup per (list, unit) -- lists are V slots, K1 rows and K2 rows --
// first drops the entries the read kernel marked as merged away (K rows a
// token already listed, key = n; V key n*n = no slot), keeping the order,
// then sorts the remaining (row, pair index) entries by row with a stable LSD
// radix sort held entirely in LDS (8-bit digits; as many passes as the
// largest row present needs).  Stability keeps every row's pairs in ascending
// (token, rank) order, so each row's gradients are summed in one fixed order
// and no float atomics are used.
// [gist.science "Fast-weight Product Key Memory", section 2, Key Technical
// Choices: gradients of slots accessed several times in a chunk are
// aggregated (averaged)]
//
// Ranking inside a wave uses ballots: the lanes holding the same digit are
// found with one ballot per digit bit, a lane's rank among them is the
// population count of the lower such lanes.  Each wave owns a contiguous run
// of 64-entry tiles and one counter per digit, so the scatter base of a
// (digit, wave) is an exclusive scan in digit-major order.  Scans run on DPP
// row shifts; rows and pair indices move together, so no pass looks a key up
// indirectly.
//
// Outputs per (list, unit): the sorted pair indices, the segments (runs of
// one row), and the segments split by length: short ones (at most kShortSeg
// pairs) get one wave of the update kernel each, long ones -- a row touched
// by dozens or hundreds of tokens -- a whole workgroup.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kBits = 8;
constexpr int kDigits = 1 << kBits;
constexpr int kSortWaves = kSortThreads / kWave;

// Inclusive scan across the wave: DPP row shifts, then row totals by readlane.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int r0 = readlane_i(x, 15), r1 = readlane_i(x, 31), r2 = readlane_i(x, 47);
  const int row = lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Exclusive scan of one int per thread across the block; *total = block sum.
__device__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int wave = threadIdx.x / kWave;
  const int incl = wave_inclusive_scan(x);
  if (lane_id() == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    sum += t;
  }
  __syncthreads();          // wave_tot may be reused right after
  *total = sum;
  return base + incl - x;
}

__device__ int block_max(int x, int* wave_tot) {
  x = max(x, xor_lane<32>(x));
  x = max(x, xor_lane<16>(x));
  x = max(x, xor_lane<8>(x));
  x = max(x, xor_lane<4>(x));
  x = max(x, xor_lane<2>(x));
  x = max(x, xor_lane<1>(x));
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) wave_tot[wave] = x;
  __syncthreads();
  int m = wave_tot[0];
#pragma unroll
  for (int w = 1; w < kSortWaves; ++w) m = m > wave_tot[w] ? m : wave_tot[w];
  __syncthreads();
  return m;
}

// Lanes of this wave holding the same digit (among `valid` lanes).
__device__ __forceinline__ unsigned long long digit_peers(int d, bool valid) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < kBits; ++bit) {
    const unsigned long long on = __ballot((d >> bit) & 1);
    peers &= ((d >> bit) & 1) ? on : ~on;
  }
  return peers;
}

}  // namespace

__global__ __launch_bounds__(kSortThreads) void kc_sort(ChunkArgs a) {
  extern __shared__ int lds[];
  const int list = blockIdx.x;   // 0 = V slots, 1 = K1 rows, 2 = K2 rows
  const int u = blockIdx.y;
  const int P = a.P;
  int* key0 = lds;                        // [P] rows (ping)
  int* idx0 = key0 + P;                   // [P] pair indices (ping)
  int* key1 = idx0 + P;                   // [P] (pong)
  int* idx1 = key1 + P;                   // [P] (pong)
  int* cnt = idx1 + P;                    // [kSortWaves][kDigits]
  int* wave_tot = cnt + kSortWaves * kDigits;   // [kSortWaves]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int lu = list * a.U + u;
  const int64_t UP = (int64_t)a.U * P;
  const int* keys = a.keys + list * UP + (int64_t)u * P;
  const int invalid_key = (list == 0) ? a.n * a.n : a.n;

  // ---- load by 64-entry tiles (wave w owns tiles [w*tpw, (w+1)*tpw)), drop
  // marked entries keeping the order, find the largest row
  const int tiles = (P + kWave - 1) / kWave;
  const int tpw = (tiles + kSortWaves - 1) / kSortWaves;
  int kept = 0, kmax = 0;
  for (int tile = wave * tpw; tile < min(tiles, (wave + 1) * tpw); ++tile) {
    const int i = tile * kWave + lane;
    const int key = i < P ? keys[i] : invalid_key;
    const bool ok = key != invalid_key;
    kept += __popcll(__ballot(ok));
    kmax = ok && key > kmax ? key : kmax;
  }
  if (lane == 0) wave_tot[wave] = kept;
  __syncthreads();
  int base = 0, Pv = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    Pv += t;
  }
  __syncthreads();
  for (int tile = wave * tpw; tile < min(tiles, (wave + 1) * tpw); ++tile) {
    const int i = tile * kWave + lane;
    const int key = i < P ? keys[i] : invalid_key;
    const bool ok = key != invalid_key;
    const unsigned long long m = __ballot(ok);
    if (ok) {
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      key0[pos] = key;
      idx0[pos] = i;
    }
    base += __popcll(m);
  }
  kmax = block_max(kmax, wave_tot);
  int bits = 0;
  while (bits < 31 && (kmax >> bits) != 0) ++bits;
  const int passes = (bits + kBits - 1) / kBits;

  // ---- LSD radix passes over the Pv kept entries
  const int vtiles = (Pv + kWave - 1) / kWave;
  const int vtpw = (vtiles + kSortWaves - 1) / kSortWaves;
  const int t_lo = wave * vtpw;
  const int t_hi = min(vtiles, t_lo + vtpw);
  int *ks = key0, *is = idx0, *kd = key1, *id = idx1;
  int* mycnt = cnt + wave * kDigits;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kBits;
    for (int i = tid; i < kSortWaves * kDigits; i += kSortThreads) cnt[i] = 0;
    __syncthreads();
    for (int tile = t_lo; tile < t_hi; ++tile) {
      const int i = tile * kWave + lane;
      const bool valid = i < Pv;
      const int d = valid ? (((unsigned)ks[i] >> shift) & (kDigits - 1)) : 0;
      const unsigned long long peers = digit_peers(d, valid);
      if (valid && (peers & ((1ull << lane) - 1ull)) == 0ull) mycnt[d] += __popcll(peers);
    }
    __syncthreads();
    {  // exclusive scan, digit-major / wave-minor: flat f = d * kSortWaves + w
      constexpr int E = kSortWaves * kDigits / kSortThreads;
      int v[E];
      int local = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = tid * E + e;
        v[e] = cnt[(f % kSortWaves) * kDigits + f / kSortWaves];
        local += v[e];
      }
      int total;
      int run = block_exclusive_scan(local, wave_tot, &total);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = tid * E + e;
        cnt[(f % kSortWaves) * kDigits + f / kSortWaves] = run;
        run += v[e];
      }
    }
    __syncthreads();
    for (int tile = t_lo; tile < t_hi; ++tile) {
      const int i = tile * kWave + lane;
      const bool valid = i < Pv;
      const int key = valid ? ks[i] : 0;
      const int d = ((unsigned)key >> shift) & (kDigits - 1);
      const unsigned long long peers = digit_peers(d, valid);
      const unsigned long long lower = peers & ((1ull << lane) - 1ull);
      const int b0 = valid ? mycnt[d] : 0;
      if (valid) {
        const int dst = b0 + __popcll(lower);
        kd[dst] = key;
        id[dst] = is[i];
      }
      if (valid && lower == 0ull) mycnt[d] = b0 + __popcll(peers);
    }
    __syncthreads();
    int* t;
    t = ks; ks = kd; kd = t;
    t = is; is = id; id = t;
  }

  // ---- segments: heads of runs of equal rows.  The pong buffers are free
  // now; segment starts go to kd[0..nseg], whose last entry may spill into
  // id[0] (kd and id are adjacent and both unused).
  int* segl = kd;
  int* sorted = a.sorted + list * UP + (int64_t)u * P;
  int* seg = a.seg_start + list * (UP + a.U) + (int64_t)u * (P + 1);
  int heads_w = 0;
  for (int tile = t_lo; tile < t_hi; ++tile) {
    const int i = tile * kWave + lane;
    const bool head = i < Pv && (i == 0 || ks[i - 1] != ks[i]);
    heads_w += __popcll(__ballot(head));
  }
  if (lane == 0) wave_tot[wave] = heads_w;
  __syncthreads();
  int hbase = 0, nseg = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    const int t = wave_tot[w];
    hbase += w < wave ? t : 0;
    nseg += t;
  }
  __syncthreads();
  for (int tile = t_lo; tile < t_hi; ++tile) {
    const int i = tile * kWave + lane;
    const bool in = i < Pv;
    const bool head = in && (i == 0 || ks[i - 1] != ks[i]);
    const unsigned long long m = __ballot(head);
    if (in) sorted[i] = is[i];
    if (head) {
      const int s = hbase + __popcll(m & ((1ull << lane) - 1ull));
      segl[s] = i;
      seg[s] = i;
    }
    hbase += __popcll(m);
  }
  if (tid == 0) {
    segl[nseg] = Pv;
    seg[nseg] = Pv;
    a.nseg[lu] = nseg;
  }
  __syncthreads();

  // ---- short / long segment lists, each in row order
  const int stiles = (nseg + kWave - 1) / kWave;
  const int stpw = (stiles + kSortWaves - 1) / kSortWaves;
  const int s_lo = wave * stpw, s_hi = min(stiles, s_lo + stpw);
  int nl = 0, ns = 0;
  for (int tile = s_lo; tile < s_hi; ++tile) {
    const int s = tile * kWave + lane;
    const bool in = s < nseg;
    const bool lng = in && segl[s + 1] - segl[s] > kShortSeg;
    nl += __popcll(__ballot(lng));
    ns += __popcll(__ballot(in && !lng));
  }
  if (lane == 0) { wave_tot[wave] = nl; cnt[wave] = ns; }
  __syncthreads();
  int lbase = 0, sbase = 0, tot_long = 0, tot_short = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    lbase += w < wave ? wave_tot[w] : 0;
    sbase += w < wave ? cnt[w] : 0;
    tot_long += wave_tot[w];
    tot_short += cnt[w];
  }
  int* long_seg = a.long_seg + list * UP + (int64_t)u * P;
  int* short_seg = a.short_seg + list * UP + (int64_t)u * P;
  for (int tile = s_lo; tile < s_hi; ++tile) {
    const int s = tile * kWave + lane;
    const bool in = s < nseg;
    const bool lng = in && segl[s + 1] - segl[s] > kShortSeg;
    const unsigned long long ml = __ballot(lng), msh = __ballot(in && !lng);
    const unsigned long long below = (1ull << lane) - 1ull;
    if (lng) long_seg[lbase + __popcll(ml & below)] = s;
    if (in && !lng) short_seg[sbase + __popcll(msh & below)] = s;
    lbase += __popcll(ml);
    sbase += __popcll(msh);
  }
  if (tid == 0) {
    a.seg_kinds[2 * lu] = tot_long;
    a.seg_kinds[2 * lu + 1] = tot_short;
  }
}

size_t kc_smem_bytes(int P) {
  return sizeof(int) * ((size_t)4 * P + (size_t)kSortWaves * kDigits + kSortWaves);
}

hipError_t launch_kc(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const size_t smem = kc_smem_bytes(a.P);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&kc_sort), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kc_smem_bytes(kSortMaxPairs));
  if (attr != hipSuccess) return attr;
  return fw_launch(kc_sort, dim3(3, a.U), dim3(kSortThreads), (uint32_t)smem, s, tm, a);
}

}  // namespace fwpkm
