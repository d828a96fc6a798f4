// KC: deterministic grouping of the chunk's (row, pair) lists.
//
// One workgroup per (list, unit) sorts the P = tokens*k pair indices of that
// unit by row key with a stable LSD radix sort held entirely in LDS
// (6-bit digits).  Stability keeps, inside each row's segment, the pairs in
// ascending (token, rank) order, so the update kernel sums every row's
// gradients in one fixed order and no float atomics are used.  It then marks
// the segment heads and writes, per list and unit, the first sorted position
// of every segment and their number.  K-row keys equal to n mark merged-away
// candidates (and V keys equal to n*n a missing slot); they sort last and form
// no segment.
// [gist.science "Fast-weight Product Key Memory", section 2, Key Technical
// Choices: gradients of slots accessed several times in a chunk are
// aggregated (averaged)]
//
// Digit ranking inside a wave uses ballots: the lanes holding the same digit
// are found with one ballot per digit bit, and a lane's rank among them is the
// population count of the lower such lanes.  Per (digit, 64-element tile)
// counts are scanned digit-major, which yields each tile's scatter base.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kDigits = 1 << kDigitBits;
constexpr int kSortWaves = kSortThreads / kWave;

// Exclusive scan of one int per thread across the 1024-thread block.
// Returns the exclusive prefix; *total receives the block sum.
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
    int v = lane < kSortWaves ? wave_tot[lane] : 0;
    int vi = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(vi, d, kWave);
      if (lane >= d) vi += y;
    }
    if (lane < kSortWaves) wave_tot[lane] = vi - v;     // exclusive wave base
    if (lane == kSortWaves - 1) wave_tot[kSortWaves] = vi;
  }
  __syncthreads();
  const int r = wave_tot[wave] + incl - x;
  *total = wave_tot[kSortWaves];
  __syncthreads();
  return r;
}

// Lanes of this wave holding the same digit (among `valid` lanes).
__device__ __forceinline__ unsigned long long digit_peers(int d, bool valid) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < kDigitBits; ++bit) {
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
  const int tiles = (P + kWave - 1) / kWave;
  int* keyl = lds;                       // [P] key of pair p
  int* buf0 = keyl + P;                  // [P] pair indices (ping)
  int* buf1 = buf0 + P;                  // [P] pair indices (pong)
  int* hist = buf1 + P;                  // [kDigits * tiles]
  int* wave_tot = hist + kDigits * tiles; // [kSortWaves + 1]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int64_t UP = (int64_t)a.U * P;
  const int* keys = a.keys + list * UP + (int64_t)u * P;

  for (int i = tid; i < P; i += kSortThreads) {
    keyl[i] = keys[i];
    buf0[i] = i;
  }
  const int bits = list == 0 ? a.key_bits_v : a.key_bits_k;
  const int passes = (bits + kDigitBits - 1) / kDigitBits;
  int* src = buf0;
  int* dst = buf1;
  __syncthreads();

  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kDigitBits;
    for (int i = tid; i < kDigits * tiles; i += kSortThreads) hist[i] = 0;
    __syncthreads();
    // counts per (digit, tile)
    for (int tile = wave; tile < tiles; tile += kSortWaves) {
      const int i = tile * kWave + lane;
      const bool valid = i < P;
      const int p = valid ? src[i] : 0;
      const int d = valid ? (((unsigned)keyl[p] >> shift) & (kDigits - 1)) : 0;
      const unsigned long long peers = digit_peers(d, valid);
      const unsigned long long lower = peers & ((1ull << lane) - 1ull);
      if (valid && lower == 0ull) hist[d * tiles + tile] = __popcll(peers);
    }
    __syncthreads();
    // exclusive scan, digit-major
    {
      const int M = kDigits * tiles;
      const int per = (M + kSortThreads - 1) / kSortThreads;
      const int beg = tid * per;
      int local = 0;
      for (int j = 0; j < per; ++j)
        if (beg + j < M) local += hist[beg + j];
      int total;
      int run = block_exclusive_scan(local, wave_tot, &total);
      for (int j = 0; j < per; ++j) {
        if (beg + j < M) {
          const int c = hist[beg + j];
          hist[beg + j] = run;
          run += c;
        }
      }
    }
    __syncthreads();
    // scatter
    for (int tile = wave; tile < tiles; tile += kSortWaves) {
      const int i = tile * kWave + lane;
      const bool valid = i < P;
      const int p = valid ? src[i] : 0;
      const int d = valid ? (((unsigned)keyl[p] >> shift) & (kDigits - 1)) : 0;
      const unsigned long long peers = digit_peers(d, valid);
      const int rank = __popcll(peers & ((1ull << lane) - 1ull));
      if (valid) dst[hist[d * tiles + tile] + rank] = p;
    }
    __syncthreads();
    int* tmp = src; src = dst; dst = tmp;
  }

  // segments: heads of runs of equal valid keys
  const int invalid_key = (list == 0) ? a.n * a.n : a.n;
  int* sorted = a.sorted + list * UP + (int64_t)u * P;
  int* seg = a.seg_start + list * (UP + a.U) + (int64_t)u * (P + 1);
  const int per = (P + kSortThreads - 1) / kSortThreads;
  const int beg = tid * per;
  int heads = 0, valids = 0;
  for (int j = 0; j < per; ++j) {
    const int i = beg + j;
    if (i < P) {
      const int key = keyl[src[i]];
      const bool ok = key != invalid_key;
      const bool head = ok && (i == 0 || keyl[src[i - 1]] != key);
      heads += head;
      valids += ok;
    }
  }
  int total;
  const int packed = block_exclusive_scan(heads | (valids << 16), wave_tot, &total);
  int hrun = packed & 0xffff;
  for (int j = 0; j < per; ++j) {
    const int i = beg + j;
    if (i < P) {
      const int key = keyl[src[i]];
      sorted[i] = src[i];
      const bool ok = key != invalid_key;
      const bool head = ok && (i == 0 || keyl[src[i - 1]] != key);
      if (head) seg[hrun++] = i;
    }
  }
  if (tid == 0) {
    const int nh = total & 0xffff;
    const int nv = total >> 16;
    seg[nh] = nv;
    a.nseg[list * a.U + u] = nh;
  }
}

size_t kc_smem_bytes(int P) {
  const int tiles = (P + kWave - 1) / kWave;
  return sizeof(int) * ((size_t)3 * P + (size_t)kDigits * tiles + kSortWaves + 1);
}

hipError_t launch_kc(const ChunkArgs& a, hipStream_t s) {
  const size_t smem = kc_smem_bytes(a.P);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&kc_sort), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kc_smem_bytes(kSortMaxPairs));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kc_sort, dim3(3, a.U), dim3(kSortThreads), smem, s, a);
  return hipGetLastError();
}

}  // namespace fwpkm
