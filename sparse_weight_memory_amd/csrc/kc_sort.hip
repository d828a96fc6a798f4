// KC: deterministic grouping of the chunk's (row, pair) lists.
//
// Lists are V slots, K1 rows and K2 rows, one of each per unit.  The rows of
// a list are split into `regions` hash classes and one workgroup handles one
// (region, list, unit): it scans the whole list once, keeps its own entries
// in their original order (dropping those the read kernel marked as merged
// away: K rows a token already listed, key n; V key n*n = no slot) and counts
// the entries of lower regions, which fixes where its output goes.  Then it
// sorts its entries by row, stably, in LDS.  A region of at most 64 entries,
// or of at most 256 whose rows span more than 8 bits, packs each (row,
// position in list order) into one 32-bit word and places every entry at the
// count of words below its own (one pass, every entry against every other);
// other regions use an LSD radix sort (8-bit digits; as many passes as the
// largest row needs).  A region of at least 512 entries whose rows need two
// or more passes first tries to rename its rows to their rank among its
// distinct rows (a hash set in LDS, then every distinct row against every
// other): with at most 256 of them -- hot rows, as in a long stream of
// clustered tokens -- one pass over the ranks gives the same order.
// Stability keeps every row's pairs in ascending (token, rank) order, so each
// row's gradient is summed in one fixed order and no float atomics are used.
// [gist.science "Fast-weight Product Key Memory", section 2, Key Technical
// Choices: gradients of slots accessed several times in a chunk are
// aggregated (averaged)]
//
// Splitting a list over several workgroups spreads the sort over many
// compute units; a row lands in exactly one region, so segments never cross
// regions and the result does not depend on the region count.
//
// Radix ranking inside a wave uses ballots: the lanes holding the same digit are
// found with one ballot per digit bit, a lane's rank among them is the
// population count of the lower such lanes.  Each wave owns a contiguous run
// of 64-entry tiles and one counter per digit, so the scatter base of a
// (digit, wave) is an exclusive scan in digit-major order.  Scans run on DPP
// row shifts; rows and pair indices move together, so no pass looks a key up
// indirectly.
//
// Outputs per region, at its offset in the (list, unit) arrays (regions
// follow one another in hash order, so a run of regions is one contiguous
// run of entries):
//   ent_row    the kept entries' rows in sorted order (a segment is a run of
//              equal rows);
//   ent_tw     their (token, weight) -- the pair's softmax weight for V, its
//              merged key coefficient for K1 / K2 -- so the update kernel
//              reads everything about an entry in one round;
//   kinds      (0, 0, offset, entries).

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kBits = 8;
constexpr int kDigits = 1 << kBits;
constexpr int kGroupThreads = kGroupWaves * kWave;
constexpr int kScanTiles = kSortMaxPairs / (kWave * kGroupWaves);   // key tiles per wave, at most
// Rank sort limits: positions in kRankPosBits bits, rows below
// 2^(32 - kRankPosBits).  Its all-pairs compares cost M^2 / 64 vector
// instructions per workgroup; past ~256 entries two radix passes are cheaper.
constexpr int kRankPosBits = 8;
constexpr int kRankMax = 1 << kRankPosBits;
constexpr int kRankBatch = 32;   // words compared per round, eight 16-byte reads in flight
constexpr int kRankPartOffset = 1024;   // partial counts after the packed words, in the counters' space
static_assert(kRankMax <= kGroupThreads, "one ranked entry per thread");
static_assert(kRankMax + kRankBatch - 1 <= kRankPartOffset, "packed words before the partial counts");
static_assert(kRankPartOffset + (kGroupWaves - 1) * kWave <= kGroupWaves * kDigits,
              "partial counts fit the counters' space");
// Renaming: a region of at least kRenameMin entries whose rows need two or
// more radix passes first maps its rows to their rank among its distinct
// rows, through a hash set of kRenameSlots rows in the counters' space;
// with at most kRenameMax distinct rows one pass then sorts the ranks.
constexpr int kRenameBits = 10;
constexpr int kRenameSlots = 1 << kRenameBits;
constexpr int kRenameMax = 256;          // = kDigits: one pass
constexpr int kRenameMin = 2 * kRenameMax;
constexpr int kRenameProbes = 32;        // longest probe run tried before giving up
constexpr int kRenameInts = kRenameMax + 8;   // row of each rank, then two control words
constexpr int kRenamePong = 3 + (kRenameMax + 4) + kRenameMax;   // alignment, distinct rows, their slots
static_assert(2 * kRenameSlots <= kGroupWaves * kDigits, "hash set and slot ranks fit the counters' space");
static_assert(kRenameMax == kDigits, "renamed rows take one pass");

// r + (w < me): the compare's carry feeds the add (two instructions).
__device__ __forceinline__ unsigned int add_if_below(unsigned int r, unsigned int w, unsigned int me) {
  asm("v_cmp_lt_u32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, 0, %0, vcc" : "+v"(r) : "v"(w), "v"(me) : "vcc");
  return r;
}

// Region of a row: multiplicative (Fibonacci) hashing, so rows that many
// tokens share spread over the regions.
__device__ __forceinline__ int region_of(int key, int bits) {
  return bits == 0 ? 0 : (int)(((unsigned)key * 0x9E3779B1u) >> (32 - bits));
}

// Exclusive scan of one int per thread across the block; *total = block sum.
// wave_tot must not be written again before the caller's next barrier.
__device__ int block_exclusive_scan(int x, int* wave_tot, int* total) {
  const int wave = threadIdx.x / kWave;
  const int incl = wave_inclusive_scan(x);
  if (lane_id() == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kGroupWaves; ++w) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    sum += t;
  }
  *total = sum;
  return base + incl - x;
}

// Lanes of this wave holding the same digit (among `valid` lanes).  Digit
// bits from `nbits` up are zero in every lane (the keys' range), so their
// ballots would change nothing and are skipped (nbits is wave-uniform).
__device__ __forceinline__ unsigned long long digit_peers(int d, bool valid, int nbits) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < kBits; ++bit) {
    if (bit >= nbits) break;
    const unsigned long long on = __ballot((d >> bit) & 1);
    peers &= ((d >> bit) & 1) ? on : ~on;
  }
  return peers;
}

__device__ __forceinline__ unsigned long long lanes_below() {
  return (1ull << lane_id()) - 1ull;
}

}  // namespace

__global__ __launch_bounds__(kGroupThreads) void kc_sort(ChunkArgs a) {
  extern __shared__ int lds[];
  const int per_unit = 3 * a.regions;
  const int item = unit_affine_item(blockIdx.x, a.U, per_unit);
  const int lr = item >> a.region_bits;   // u * 3 + list (regions is a power of two)
  const int u = lr / 3;
  const int list = lr - 3 * u;            // 0 = V slots, 1 = K1 rows, 2 = K2 rows
  const int region = item & (a.regions - 1);
  const int P = a.P;
  int* key0 = lds;                        // [P] rows (ping)
  int* idx0 = key0 + P;                   // [P] pair indices (ping)
  int* key1 = idx0 + P;                   // [P] (pong)
  int* idx1 = key1 + P;                   // [P] (pong)
  int* cnt = idx1 + P;                    // [kGroupWaves][kDigits]
  int* red = cnt + kGroupWaves * kDigits; // [3][kGroupWaves]
  int* rowof = red + 3 * kGroupWaves;     // [kRenameMax] row of each rank, [+0, +1] control words

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int64_t lbase = ((int64_t)list * a.U + u) * P;   // this (list, unit) in [3, U, P]
  const int* keys = a.keys + lbase;
  const int invalid_key = (list == 0) ? a.n * a.n : a.n;

  // ---- scan the list: wave w owns key tiles [w*tpw, (w+1)*tpw); all loads
  // are issued before any is used
  const int tiles = (P + kWave - 1) / kWave;
  const int tpw = (tiles + kGroupWaves - 1) / kGroupWaves;   // <= kScanTiles
  int kreg[kScanTiles];
#pragma unroll
  for (int j = 0; j < kScanTiles; ++j) {
    const int i = (wave * tpw + j) * kWave + lane;
    kreg[j] = (j < tpw && i < P) ? keys[i] : invalid_key;
  }
  // (tiles past tpw are skipped by a wave-uniform test, not a break: a loop
  // that can leave early is not unrolled, and kreg[j] at a run-time j is an
  // indexed register access, ~250 cycles a tile on the shared scalar unit)
  int kept = 0, below = 0, kmax = 0;
#pragma unroll
  for (int j = 0; j < kScanTiles; ++j) {
    if (j < tpw) {
      const int key = kreg[j];
      const bool ok = key != invalid_key;
      const int rg = region_of(key, a.region_bits);
      const bool mine = ok && rg == region;
      below += __popcll(__ballot(ok && rg < region));
      kept += __popcll(__ballot(mine));
      kmax = mine && key > kmax ? key : kmax;
    }
  }
  kmax = max(kmax, xor_lane<32>(kmax));
  kmax = max(kmax, xor_lane<16>(kmax));
  kmax = max(kmax, xor_lane<8>(kmax));
  kmax = max(kmax, xor_lane<4>(kmax));
  kmax = max(kmax, xor_lane<2>(kmax));
  kmax = max(kmax, xor_lane<1>(kmax));
  if (lane == 0) {
    red[wave] = kept;
    red[kGroupWaves + wave] = below;
    red[2 * kGroupWaves + wave] = kmax;
  }
  __syncthreads();
  int base = 0, M = 0, off = 0;
  kmax = 0;
#pragma unroll
  for (int w = 0; w < kGroupWaves; ++w) {
    const int t = red[w];
    base += w < wave ? t : 0;
    M += t;
    off += red[kGroupWaves + w];
    kmax = max(kmax, red[2 * kGroupWaves + w]);
  }
  int4* kinds = a.kinds + ((int64_t)list * a.U + u) * a.regions + region;
  if (M == 0) {                     // block-uniform
    if (tid == 0) *kinds = make_int4(0, 0, off, 0);   // no entries
    return;
  }
  // regions of at most kRankMax entries whose rows need two or more radix
  // passes, and regions of at most 64 entries, are sorted by ranking (below);
  // their packed (row, position) words use the radix counters' space
  // (against one radix pass, ranking pays only for the smallest regions)
  const bool by_rank = kmax < (1 << (32 - kRankPosBits)) &&
                       (M <= kWave || (M <= kRankMax && kmax >= kDigits));
  unsigned int* packed = reinterpret_cast<unsigned int*>(cnt);
#pragma unroll
  for (int j = 0; j < kScanTiles; ++j) {
    if (j < tpw) {                                   // wave-uniform (see above)
      const int key = kreg[j];
      const bool mine = key != invalid_key && region_of(key, a.region_bits) == region;
      const unsigned long long m = __ballot(mine);
      if (mine) {
        const int pos = base + __popcll(m & lanes_below());
        key0[pos] = key;
        idx0[pos] = (wave * tpw + j) * kWave + lane;
        if (by_rank) packed[pos] = ((unsigned int)key << kRankPosBits) | (unsigned int)pos;
      }
      base += __popcll(m);
    }
  }
  int* mycnt = cnt + wave * kDigits;   // only this wave counts into / scatters from it
  // radix passes the rows need, and whether to rename them first (below)
  int bits = bit_length(kmax);
  int passes = (bits + kBits - 1) / kBits;
  const bool try_rename = !by_rank && passes >= 2 && M >= kRenameMin && P >= kRenamePong;   // block-uniform
  // renaming: a hash set of rows in the counters' space, the row of each
  // rank, two control words, and the distinct rows (padded to whole int4
  // reads, 16-byte aligned) and their slots in the pong buffer (P ints,
  // at least kRenamePong)
  int* tab = cnt;                                            // [kRenameSlots] row, -1 = empty
  int* rank_of = cnt + kRenameSlots;                         // [kRenameSlots] rank of the slot's row
  int* ctl = rowof + kRenameMax;                             // distinct rows found, overflow
  int* drow = key1 + ((4 - (int)((reinterpret_cast<uintptr_t>(key1) >> 2) & 3)) & 3);   // [kRenameMax + 4]
  int* dslot = drow + kRenameMax + 4;                        // [kRenameMax]
  if (by_rank) {
    if (tid < kRankBatch - 1) packed[M + tid] = 0xFFFFFFFFu;   // pad to whole batches; never below a real word
  } else if (try_rename) {
    for (int q = tid; q < kRenameSlots; q += kGroupThreads) tab[q] = -1;
    for (int q = tid; q < kRenameMax + 4; q += kGroupThreads) drow[q] = 0x7FFFFFFF;
    if (tid == 0) {
      ctl[0] = 0;
      ctl[1] = 0;
    }
  } else {
    for (int i = lane; i < kDigits; i += kWave) mycnt[i] = 0;
  }
  __syncthreads();

  // wave w owns tiles [t_lo, t_hi) of the M kept entries
  const int vtiles = (M + kWave - 1) / kWave;
  const int vtpw = (vtiles + kGroupWaves - 1) / kGroupWaves;
  const int t_lo = wave * vtpw;
  const int t_hi = min(vtiles, t_lo + vtpw);
  int *ks = key0, *is = idx0, *kd = key1, *id = idx1;
  bool renamed = false;
  if (by_rank) {
    // ---- rank sort: the words are distinct and ordered as (row, position),
    // so an entry's place in the stable order is the number of words below
    // its own.  Every wave takes one 64-entry tile and one share of the
    // word batches (all lanes read the same words: LDS broadcast reads);
    // with fewer tiles than waves, the shares' counts meet in LDS.
    const int rtiles = (M + kWave - 1) / kWave;
    const int shares = kGroupWaves / rtiles;                // >= 1
    const int rtile = wave % rtiles, share = wave / rtiles;
    const int i = rtile * kWave + lane;
    const int nb = (M + kRankBatch - 1) / kRankBatch;
    // wave-uniform bounds (scalar loop)
    const int b_lo = __builtin_amdgcn_readfirstlane(share * nb / shares);
    const int b_hi = __builtin_amdgcn_readfirstlane((share + 1) * nb / shares);
    int* part = cnt + kRankPartOffset;                      // [shares][M] partial counts
    int rank = 0;
    if (share < shares) {
      const unsigned int me = i < M ? packed[i] : 0u;
      const uint4* p4 = reinterpret_cast<const uint4*>(packed);
      unsigned int r[kRankBatch / 4] = {};
      for (int bb = b_lo; bb < b_hi; ++bb) {
        uint4 v[kRankBatch / 4];
#pragma unroll
        for (int q = 0; q < kRankBatch / 4; ++q) v[q] = p4[bb * (kRankBatch / 4) + q];   // all in flight
#pragma unroll
        for (int q = 0; q < kRankBatch / 4; ++q) {
          r[q] = add_if_below(r[q], v[q].x, me);
          r[q] = add_if_below(r[q], v[q].y, me);
          r[q] = add_if_below(r[q], v[q].z, me);
          r[q] = add_if_below(r[q], v[q].w, me);
        }
      }
#pragma unroll
      for (int q = 0; q < kRankBatch / 4; ++q) rank += (int)r[q];
      if (shares > 1 && share > 0 && i < M) part[(share - 1) * M + i] = rank;
    }
    if (shares > 1) __syncthreads();                        // block-uniform
    if (share == 0 && i < M) {
      for (int sh = 1; sh < shares; ++sh) rank += part[(sh - 1) * M + i];
      key1[rank] = key0[i];
      idx1[rank] = idx0[i];
    }
    __syncthreads();
    ks = key1; is = idx1; kd = key0; id = idx0;
  } else {
  // ---- rename the rows to their rank among the region's distinct rows
  // (hot rows: few distinct rows, many entries).  Each entry's row goes
  // into a hash set (linear probing, compare-and-swap; the set of distinct
  // rows found does not depend on the order of insertion); the distinct
  // rows are ranked by value, each against all, so ranks keep the rows'
  // order and one stable pass over the ranks gives exactly the order the
  // passes over the rows would.  More than kRenameMax distinct rows, or a
  // probe run longer than kRenameProbes, leaves the rows as they are (once
  // the count has passed the limit every lane stops at its next probe and
  // every wave at its next tile, so regions of many distinct rows give up
  // early).
  if (try_rename) {
    int* eslot = id;                                         // [M] slot of each entry
    for (int tile = t_lo; tile < t_hi; ++tile) {
      // too many distinct rows already: renaming is off, this wave stops
      if (__builtin_amdgcn_readfirstlane(*(volatile int*)&ctl[0]) > kRenameMax) break;
      const int i = tile * kWave + lane;
      if (i < M) {
        const int r = ks[i];
        int h = (int)(((unsigned)r * 0x85EBCA6Bu) >> (32 - kRenameBits));
        int slot = -1;
        for (int probe = 0; probe < kRenameProbes; ++probe) {
          if (*(volatile int*)&ctl[0] > kRenameMax) break;   // renaming is off: stop at once
          const int old = atomicCAS(&tab[h], -1, r);
          if (old == -1) {
            const int d = atomicAdd(&ctl[0], 1);
            if (d < kRenameMax) {
              drow[d] = r;
              dslot[d] = h;
            }
            slot = h;
            break;
          }
          if (old == r) {
            slot = h;
            break;
          }
          h = (h + 1) & (kRenameSlots - 1);
        }
        if (slot < 0) ctl[1] = 1;
        eslot[i] = slot;
      }
    }
    __syncthreads();
    const int D = ctl[0];
    if (D <= kRenameMax && ctl[1] == 0) {                    // block-uniform
      if (tid < D) {
        const int me = drow[tid];
        const int4* d4 = reinterpret_cast<const int4*>(drow);
        int rk = 0;
        for (int j = 0; j < (D + 3) / 4; ++j) {              // pads sort last
          const int4 w = d4[j];
          rk += (w.x < me) + (w.y < me) + (w.z < me) + (w.w < me);
        }
        rank_of[dslot[tid]] = rk;
        rowof[rk] = me;
      }
      __syncthreads();
      for (int tile = t_lo; tile < t_hi; ++tile) {
        const int i = tile * kWave + lane;
        if (i < M) ks[i] = rank_of[eslot[i]];
      }
      // ranks take bitlen(D - 1) bits; one distinct row is sorted already
      bits = min(kBits, bit_length(D - 1));
      passes = D > 1 ? 1 : 0;
      renamed = true;
      __syncthreads();         // every wave has read the slot ranks before the counters are cleared
    }
    for (int i = lane; i < kDigits; i += kWave) mycnt[i] = 0;   // the set used the counters
    __syncthreads();
  }

  // ---- LSD radix passes over the M kept entries
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = pass * kBits;
    const int nbits = min(kBits, bits - shift);   // digit bits any key of this pass can have
    for (int tile = t_lo; tile < t_hi; ++tile) {
      const int i = tile * kWave + lane;
      const bool valid = i < M;
      const int d = valid ? (((unsigned)ks[i] >> shift) & (kDigits - 1)) : 0;
      const unsigned long long peers = digit_peers(d, valid, nbits);
      if (valid && (peers & lanes_below()) == 0ull) mycnt[d] += __popcll(peers);
    }
    __syncthreads();
    {  // exclusive scan, digit-major / wave-minor: flat f = d * kGroupWaves + w
      constexpr int E = kGroupWaves * kDigits / kGroupThreads;
      int v[E];
      int local = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = tid * E + e;
        v[e] = cnt[(f % kGroupWaves) * kDigits + f / kGroupWaves];
        local += v[e];
      }
      int total;
      int run = block_exclusive_scan(local, red, &total);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = tid * E + e;
        cnt[(f % kGroupWaves) * kDigits + f / kGroupWaves] = run;
        run += v[e];
      }
    }
    __syncthreads();
    for (int tile = t_lo; tile < t_hi; ++tile) {
      const int i = tile * kWave + lane;
      const bool valid = i < M;
      const int key = valid ? ks[i] : 0;
      const int d = ((unsigned)key >> shift) & (kDigits - 1);
      const unsigned long long peers = digit_peers(d, valid, nbits);
      const unsigned long long lower = peers & lanes_below();
      const int b0 = valid ? mycnt[d] : 0;
      if (valid) {
        const int dst = b0 + __popcll(lower);
        kd[dst] = key;
        id[dst] = is[i];
      }
      if (valid && lower == 0ull) mycnt[d] = b0 + __popcll(peers);
    }
    for (int i = lane; i < kDigits; i += kWave) mycnt[i] = 0;   // for the next pass
    __syncthreads();
    int* t;
    t = ks; ks = kd; kd = t;
    t = is; is = id; id = t;
  }
  }

  if (tid == 0) *kinds = make_int4(0, 0, off, M);

  // ---- entries in sorted order: row, then (token, weight or coefficient)
  // of the pair; the weight lookups of a wave go out together
  int* erow = a.ent_row + lbase + off;
  int2* etw = a.ent_tw + lbase + off;
  const float* wsrc = list == 0 ? a.sel_w + (int64_t)u * P
                                : a.coef + (int64_t)(list - 1) * a.U * P + (int64_t)u * P;
  constexpr int kOutTiles = kScanTiles;
  float wv[kOutTiles];
  int pv[kOutTiles];
#pragma unroll
  for (int j = 0; j < kOutTiles; ++j) {
    const int i = (t_lo + j) * kWave + lane;
    pv[j] = (t_lo + j < t_hi && i < M) ? is[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < kOutTiles; ++j) wv[j] = wsrc[pv[j]];
#pragma unroll
  for (int j = 0; j < kOutTiles; ++j) {
    const int i = (t_lo + j) * kWave + lane;
    if (t_lo + j < t_hi && i < M) {
      const int row = renamed ? rowof[ks[i]] : ks[i];
      erow[i] = row;
      device_check(a, row == keys[pv[j]], kChkEntry);        // the pair's own row
      etw[i] = make_int2(token_of(pv[j], a.k), __float_as_int(wv[j]));
    }
  }
}

int group_regions(int units) {
  int r = 1;
  while (r < 64 && 3 * units * r * 2 <= 256) r *= 2;
  return r;
}

size_t kc_smem_bytes(int P) {
  return sizeof(int) * ((size_t)4 * P + (size_t)kGroupWaves * kDigits + 3 * kGroupWaves + kRenameInts);
}

hipError_t launch_kc(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const size_t smem = kc_smem_bytes(a.P);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&kc_sort), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kc_smem_bytes(kSortMaxPairs));
  if (attr != hipSuccess) return attr;
  // unit-major (region fastest), see unit_affine_item
  return fw_launch(kc_sort, dim3((unsigned)(a.regions * 3 * a.U)), dim3(kGroupThreads), (uint32_t)smem, s, tm, a);
}

}  // namespace fwpkm
