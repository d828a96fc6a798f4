// KC: deterministic grouping of the chunk's (row, pair) lists.
//
// One workgroup per (list, unit) -- lists are V slots, K1 rows and K2 rows --
// first drops the entries the read kernel marked as merged away (K rows a
// token already listed, key = n; V key n*n = no slot), keeping the order,
// then sorts the remaining pair indices by row key with a stable LSD radix
// sort held entirely in LDS (8-bit digits; as many passes as the largest key
// present needs).  Stability keeps every row's pairs in ascending
// (token, rank) order, so each row's gradients are summed in one fixed order
// and no float atomics are used.
// [gist.science "Fast-weight Product Key Memory", section 2, Key Technical
// Choices: gradients of slots accessed several times in a chunk are
// aggregated (averaged)]
//
// Outputs per (list, unit): the sorted pair indices, the segments (runs of
// one row), and the segments split by length: short ones (at most kShortSeg
// pairs) get one wave of the update kernel each, long ones -- a row touched
// by dozens or hundreds of tokens -- a whole workgroup.
//
// Ranking inside a wave uses ballots: the lanes holding the same digit are
// found with one ballot per digit bit, a lane's rank among them is the
// population count of the lower such lanes.  Each wave owns a contiguous run
// of 64-element tiles and one counter per digit, so the scatter base of a
// (digit, wave) is an exclusive scan in digit-major order.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kBits = 8;
constexpr int kDigits = 1 << kBits;
constexpr int kSortWaves = kSortThreads / kWave;

// Exclusive scan of one int per thread across the block; *total = block sum.
__device__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int incl = x;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < kSortWaves ? wave_tot[lane] : 0;
    int vi = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(vi, d, kWave);
      if (lane >= d) vi += y;
    }
    if (lane < kSortWaves) wave_tot[lane] = vi - v;
    if (lane == kSortWaves - 1) wave_tot[kSortWaves] = vi;
  }
  __syncthreads();
  const int r = wave_tot[wave] + incl - x;
  *total = wave_tot[kSortWaves];
  __syncthreads();
  return r;
}

__device__ int block_max(int x, int* wave_tot) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) {
    const int y = __shfl_xor(x, d, kWave);
    x = x > y ? x : y;
  }
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) wave_tot[wave] = x;
  __syncthreads();
  int m = wave_tot[0];
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
  int* keyl = lds;                        // [P] key of pair p
  int* buf0 = keyl + P;                   // [P] pair indices (ping)
  int* buf1 = buf0 + P;                   // [P] pair indices (pong)
  int* segl = buf1 + P;                   // [P + 1] segment starts
  int* cnt = segl + P + 1;                // [kSortWaves][kDigits]
  int* wave_tot = cnt + kSortWaves * kDigits;   // [kSortWaves + 1]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int lu = list * a.U + u;
  const int64_t UP = (int64_t)a.U * P;
  const int* keys = a.keys + list * UP + (int64_t)u * P;
  const int invalid_key = (list == 0) ? a.n * a.n : a.n;

  // ---- load, drop marked entries (order kept), find the largest key
  const int per = (P + kSortThreads - 1) / kSortThreads;
  const int beg = tid * per;
  int nvalid = 0, kmax = 0;
  for (int j = 0; j < per; ++j) {
    const int p = beg + j;
    if (p < P) {
      const int key = keys[p];
      keyl[p] = key;
      if (key != invalid_key) { ++nvalid; kmax = key > kmax ? key : kmax; }
    }
  }
  int Pv;
  int pos = block_exclusive_scan(nvalid, wave_tot, &Pv);
  for (int j = 0; j < per; ++j) {
    const int p = beg + j;
    if (p < P && keyl[p] != invalid_key) buf0[pos++] = p;
  }
  kmax = block_max(kmax, wave_tot);
  int bits = 0;
  while (bits < 31 && (kmax >> bits) != 0) ++bits;
  const int passes = (bits + kBits - 1) / kBits;

  // ---- LSD radix passes over the Pv valid entries
  const int tiles = (Pv + kWave - 1) / kWave;
  const int tpw = (tiles + kSortWaves - 1) / kSortWaves;     // tiles per wave
  const int t_lo = wave * tpw;
  const int t_hi = min(tiles, t_lo + tpw);
  int* src = buf0;
  int* dst = buf1;
  int* mycnt = cnt + wave * kDigits;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kBits;
    for (int i = tid; i < kSortWaves * kDigits; i += kSortThreads) cnt[i] = 0;
    __syncthreads();
    for (int tile = t_lo; tile < t_hi; ++tile) {
      const int i = tile * kWave + lane;
      const bool valid = i < Pv;
      const int p = valid ? src[i] : 0;
      const int d = valid ? (((unsigned)keyl[p] >> shift) & (kDigits - 1)) : 0;
      const unsigned long long peers = digit_peers(d, valid);
      if (valid && (peers & ((1ull << lane) - 1ull)) == 0ull) mycnt[d] += __popcll(peers);
    }
    __syncthreads();
    {  // exclusive scan, digit-major / wave-minor
      constexpr int M = kSortWaves * kDigits;
      constexpr int E = M / kSortThreads;
      int v[E];
      int local = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = tid * E + e;               // f = d * kSortWaves + w
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
      const int p = valid ? src[i] : 0;
      const int d = valid ? (((unsigned)keyl[p] >> shift) & (kDigits - 1)) : 0;
      const unsigned long long peers = digit_peers(d, valid);
      const unsigned long long lower = peers & ((1ull << lane) - 1ull);
      const int base = valid ? mycnt[d] : 0;
      if (valid) dst[base + __popcll(lower)] = p;
      if (valid && lower == 0ull) mycnt[d] = base + __popcll(peers);
    }
    __syncthreads();
    int* tmp = src; src = dst; dst = tmp;
  }

  // ---- segments: heads of runs of equal keys
  int* sorted = a.sorted + list * UP + (int64_t)u * P;
  int* seg = a.seg_start + list * (UP + a.U) + (int64_t)u * (P + 1);
  const int pv_per = (Pv + kSortThreads - 1) / kSortThreads;
  const int vbeg = tid * pv_per;
  int heads = 0;
  for (int j = 0; j < pv_per; ++j) {
    const int i = vbeg + j;
    if (i < Pv) heads += (i == 0 || keyl[src[i - 1]] != keyl[src[i]]);
  }
  int nseg;
  int hrun = block_exclusive_scan(heads, wave_tot, &nseg);
  for (int j = 0; j < pv_per; ++j) {
    const int i = vbeg + j;
    if (i < Pv) {
      sorted[i] = src[i];
      if (i == 0 || keyl[src[i - 1]] != keyl[src[i]]) { segl[hrun] = i; seg[hrun] = i; ++hrun; }
    }
  }
  if (tid == 0) {
    segl[nseg] = Pv;
    seg[nseg] = Pv;
    a.nseg[lu] = nseg;
  }
  __syncthreads();

  // ---- short segments (at most kShortSeg pairs: one wave) and long ones (a
  // whole update workgroup), each listed in key order
  const int sg_per = (nseg + kSortThreads - 1) / kSortThreads;
  const int sbeg = tid * sg_per;
  int n_long = 0, n_short = 0;
  for (int j = 0; j < sg_per; ++j) {
    const int s = sbeg + j;
    if (s < nseg) {
      if (segl[s + 1] - segl[s] > kShortSeg) ++n_long; else ++n_short;
    }
  }
  int totals;
  const int packed = block_exclusive_scan(n_long | (n_short << 16), wave_tot, &totals);
  int lrun = packed & 0xffff, srun = packed >> 16;
  int* long_seg = a.long_seg + list * UP + (int64_t)u * P;
  int* short_seg = a.short_seg + list * UP + (int64_t)u * P;
  for (int j = 0; j < sg_per; ++j) {
    const int s = sbeg + j;
    if (s < nseg) {
      if (segl[s + 1] - segl[s] > kShortSeg) long_seg[lrun++] = s; else short_seg[srun++] = s;
    }
  }
  if (tid == 0) {
    a.seg_kinds[2 * lu] = totals & 0xffff;
    a.seg_kinds[2 * lu + 1] = totals >> 16;
  }
}

size_t kc_smem_bytes(int P) {
  return sizeof(int) * ((size_t)4 * P + 1 + (size_t)kSortWaves * kDigits + kSortWaves + 1);
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
