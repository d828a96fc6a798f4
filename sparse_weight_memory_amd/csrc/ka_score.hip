// KA: sub-key scoring on the matrix cores, with the per-half top-k fused in.
//
// For every unit, query half h, token t and sub-key i this computes an
// ordering key o_h[t, i] whose ascending order is best-first:
//   IDW  o = ||K_h[i]||^2 - 2 q_h[t].K_h[i]   (= ||q_h - K_h[i]||^2 - ||q_h||^2)
//   dot  o = -(q_h[t].K_h[i])
// and keeps, per key block, the k best (o asc, index asc).  The query's own
// norm ||q_h||^2 is common to every candidate of a half, so it is kept apart
// (qnorm) and added back only for the weights.
// [gist.science "Fast-weight Product Key Memory", section 2: sub-key
// codebooks K(1), K(2) scored in O(sqrt N), IDW score -log(eps+||q-K||^2);
// agifrontier tutorial, Product Key addressing: query split in two halves]
//
// The q.K contraction is a dense [keys x d_h] x [d_h x tokens] product per
// unit and half: it runs on v_mfma_f32_16x16x4_f32.  A workgroup of 16 waves
// owns (unit, half, key block, 16-token tile) with the tile's queries staged
// in LDS.  The key block (64, 128 or 256 keys) is chosen per launch so that
// small chunks still spread over the whole chip: wave w multiplies key tile
// (w mod blk/16) over its share of the dims; dim shares are summed in LDS.
// Each wave stages its own 16 key rows through a private LDS slice, 64 (or,
// for d_h > 256, 32) dims at a time, loaded with whole lines (a wave-wide
// load of matrix operands straight from memory would touch 16 key rows at
// once, which the load path serves at a fraction of its rate); two (four)
// chunks are in flight in registers, two in LDS.  With no barrier inside the
// contraction, the waves of a SIMD drift apart and one's LDS traffic overlaps
// another's matrix work.
// Key norms are summed in fp32 beside the contraction (on this chip fp32
// matrix instructions share the vector issue, so every extra instruction in
// that loop costs time): their rounding, ~1e-7 of ||K||^2, stays well below
// the dot product's and the 1e-6 relative gap at which candidates count as
// tied.
//
// Selection, one wave per token, on packed 64-bit (value, index) keys: a
// bitonic sort of the first 64 candidates gives a threshold (the k-th best);
// the remaining candidates are filtered against it with one ballot per 64,
// the few that pass are compacted into LDS, and a bitonic sort of the k best
// plus the survivors (over 16, 32 or 64 lanes, whichever holds them) gives
// the block's top-k.  Every step orders by (value, index), which is unique,
// so the result is deterministic.
// Work items are laid out so that the token tiles sharing one key block run
// on one XCD (workgroup i is dispatched to XCD i % 8), which keeps the block's
// keys in that XCD's L2.

#include <algorithm>

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kScoreWaves = 16;
constexpr int kMaxBlk = 256;       // largest key block
constexpr int kStageRows = kScoreWaves * 16;              // (dim share, key) rows = 256

// kDimChunk dims of every key row are staged in LDS at a time (64 when it
// fits, else 32); kPrefetch chunks are in flight in registers.
template <int kDimChunk, int kPrefetch>
struct Staging {
  static constexpr int kKPitch = kDimChunk + 4;                  // floats per staged row (pad)
  static constexpr int kStageF4 = 16 * kDimChunk / 4 / kWave;    // float4 per lane per chunk
  static constexpr int kLanesPerRow = kDimChunk / 4;             // one float4 each
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
};

// Chunks of DC dims per dim share, rounded up to a multiple of the ring
// depth PF (the extra chunks hold zero keys).
template <int DC, int PF>
__host__ __device__ inline int ka_chunks(int half, int blk) {
  const int ndq = kScoreWaves / (blk / 16);
  const int share = ((half + 16 * ndq - 1) / (16 * ndq)) * 16;
  const int nchunks = (share + DC - 1) / DC;
  return (nchunks + PF - 1) / PF * PF;
}

// Width of a staged query row: every dim a chunk of any dim share may touch
// (columns past d_h are zero), so operand reads need no bounds test.
template <int DC, int PF>
__host__ __device__ inline int ka_query_width(int half, int blk) {
  const int ndq = kScoreWaves / (blk / 16);
  const int share = ((half + 16 * ndq - 1) / (16 * ndq)) * 16;
  return (ndq - 1) * share + ka_chunks<DC, PF>(half, blk) * DC;
}

// kFull: every multiplied chunk lies inside its dim share and d_h (the
// shares tile d_h in whole chunks, and no ring padding is multiplied), so
// the staging loads need no mask.
template <int kDimChunk, int kPrefetch, bool kFull>
__global__ __launch_bounds__(kScoreWaves * kWave) void ka_score_topk(ChunkArgs a) {
  constexpr int kKPitch = Staging<kDimChunk, kPrefetch>::kKPitch;
  constexpr int kStageF4 = Staging<kDimChunk, kPrefetch>::kStageF4;
  constexpr int kLanesPerRow = Staging<kDimChunk, kPrefetch>::kLanesPerRow;
  constexpr int kRowsPerLoad = Staging<kDimChunk, kPrefetch>::kRowsPerLoad;
  extern __shared__ float smem[];
  const int half = a.half;
  const int blk = a.key_block;             // 64, 128 or 256
  const int nkt = blk / 16;                // key tiles per block
  const int ndq = kScoreWaves / nkt;       // dim shares per key tile
  const int qwidth = ka_query_width<kDimChunk, kPrefetch>(half, blk);
  const int qpitch = qwidth + 4;
  float* qs = smem;                                      // [16][qpitch]
  float* kst = qs + kTokTile * qpitch;                   // [16 waves][2][16][kKPitch] staged keys
  double* knp = reinterpret_cast<double*>(kst + 2 * kStageRows * kKPitch);  // [ndq][blk]
  // after the contraction the staging buffers are free:
  float* part = kst;                                     // [ndq][16][blk + 1]
  float* sc = part;                                      // [16][blk + 1], reuses part[0]
  skey* surv = reinterpret_cast<skey*>(kst + kStageRows * kKPitch);   // [16][blk] survivors

  const int ntt = (a.T + kTokTile - 1) / kTokTile;
  const int total = a.U * 2 * a.nblk * ntt;
  const int per_xcd = (total + 7) / 8;
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L >= total) return;
  const int tt = L % ntt;
  int rest = L / ntt;
  const int kb = rest % a.nblk;
  rest /= a.nblk;
  const int h = rest % 2;
  const int u = rest / 2;
  const int b = u / a.H, hh = u % a.H;
  const int t0 = tt * kTokTile;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();

  // ---- geometry: wave (kt, dq) = key tile kt over dim share dq
  const int kt = wave % nkt;
  const int dq = wave / nkt;
  const int row = lane & 15;          // A row (key) / B column (token)
  const int quad = lane >> 4;         // 4-dim group inside a 16-dim step
  const int share = ((half + 16 * ndq - 1) / (16 * ndq)) * 16;   // dims per share
  const int steps = share / 16;
  const int nchunks = (share + kDimChunk - 1) / kDimChunk;      // chunks holding data
  const int nchunks_p = ka_chunks<kDimChunk, kPrefetch>(half, blk); // chunks multiplied
  const float* kbase = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + (int64_t)hh * a.n * half;

  // ---- key staging, private to each wave: chunk c holds the wave's 16 key
  // rows over dims [dq*share + c*kDimChunk, +kDimChunk).  The wave loads it
  // with whole lines (kLanesPerRow consecutive lanes per row) and transposes
  // it through its own LDS slice into the matrix-operand layout, so waves
  // never wait for each other inside the contraction.  kPrefetch chunks are
  // in flight in a register ring; every ring load is issued (chunks past the
  // end read a valid address and are masked to zero), so the loop body is
  // the same each time and the compiler waits only for the chunk it stores.
  float* wbuf = kst + wave * 2 * 16 * kKPitch;           // [2][16][kKPitch]
  float4 stg[kPrefetch][kStageF4];
  // per-lane parts of the staging addresses, fixed for the whole loop.  Rows
  // past n read row 0 instead (their scores are discarded); dims past the
  // share or d_h are masked to zero, so they add nothing to a dot product
  // or a norm.
  const int lane_ds = (lane % kLanesPerRow) * 4;                 // dim offset inside a chunk
  const int ds_lim = min(share, half - dq * share);              // dims of this share that exist
  int lane_off[kStageF4];
#pragma unroll
  for (int j = 0; j < kStageF4; ++j) {
    const int gk = kb * blk + kt * 16 + j * kRowsPerLoad + lane / kLanesPerRow;
    lane_off[j] = (gk < a.n ? gk : 0) * half + min(dq * share + lane_ds, half - 4);
  }
  auto stage_load = [&](float4 (&dst)[kStageF4], int c) {
    if constexpr (kFull) {
      // ring loads past the last chunk re-read chunk 0 (never multiplied)
      const int cofs = c < nchunks ? c * kDimChunk : 0;
#pragma unroll
      for (int j = 0; j < kStageF4; ++j) {
        // through the native vector type: a copy of the float4 struct would
        // go through memory
        const v4f v = *reinterpret_cast<const v4f*>(kbase + lane_off[j] + cofs);
        dst[j] = make_float4(v.x, v.y, v.z, v.w);
      }
      return;
    }
    const bool ok = c < nchunks && c * kDimChunk + lane_ds < ds_lim;
    const unsigned int m = ok ? 0xFFFFFFFFu : 0u;    // masked, so the load is never skipped
    const int cofs = ok ? c * kDimChunk : 0;
#pragma unroll
    for (int j = 0; j < kStageF4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(kbase + lane_off[j] + cofs);
      dst[j] = make_float4(__uint_as_float(__float_as_uint(v.x) & m), __uint_as_float(__float_as_uint(v.y) & m),
                           __uint_as_float(__float_as_uint(v.z) & m), __uint_as_float(__float_as_uint(v.w) & m));
    }
  };
  auto stage_store = [&](const float4 (&src)[kStageF4], int c) {
    float* buf = wbuf + (c & 1) * 16 * kKPitch;
#pragma unroll
    for (int j = 0; j < kStageF4; ++j) {
      const int r = j * kRowsPerLoad + lane / kLanesPerRow;
      *reinterpret_cast<float4*>(&buf[r * kKPitch + (lane % kLanesPerRow) * 4]) = src[j];
    }
  };
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) stage_load(stg[i], i);   // in flight while queries are staged

  // ---- stage the 16-token query tile (this half) in LDS
  const int half4 = half >> 2;
  const int qw4 = qwidth >> 2;
  for (int e = tid; e < kTokTile * qw4; e += kScoreWaves * kWave) {
    const int r = e / qw4, c4 = e - r * qw4;
    const int t = t0 + r;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < a.T && c4 < half4) {
      const float* qrow = a.q + ((int64_t)(b * a.T + t) * a.H + hh) * a.dqk + h * half;
      x = reinterpret_cast<const float4*>(qrow)[c4];
    }
    *reinterpret_cast<float4*>(&qs[r * qpitch + c4 * 4]) = x;
  }
  stage_store(stg[0], 0);
  stage_load(stg[0], kPrefetch);
  __syncthreads();

  // ---- query norms (fp64 sums), once per token and half; wave w <-> token w
  if (kb == 0 && t0 + wave < a.T) {
    double s = 0.0;
    for (int d = lane; d < half; d += kWave) {
      const double x = qs[wave * qpitch + d];
      s += x * x;
    }
    s = wave_sum_d(s);
    if (lane == 0) a.qnorm[((int64_t)u * a.T + t0 + wave) * 2 + h] = (float)s;
  }

  // ---- scores.  Two independent accumulator chains (x,y and z,w components
  // of each step); one barrier per staged chunk.
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  float ksq = 0.f;     // key norm partial (fp32: its rounding is far below the dot product's)
  const float* arow_base = &qs[row * qpitch + dq * share];
  auto mfma_chunk = [&](int c) {
    const float* krow_s = wbuf + (c & 1) * 16 * kKPitch + row * kKPitch;
#pragma unroll
    for (int j = 0; j < kDimChunk / 16; ++j) {
      // staged key dims outside this share (or past d_h) are zero, so the
      // query operand is read unguarded from the zero-padded row
      const int ds = (c * (kDimChunk / 16) + j) * 16 + quad * 4;   // dim inside the share
      const float4 ak = *reinterpret_cast<const float4*>(&krow_s[j * 16 + quad * 4]);
      const float4 bq = *reinterpret_cast<const float4*>(&arow_base[ds]);
      ksq = fmaf(ak.x, ak.x, ksq); ksq = fmaf(ak.y, ak.y, ksq);
      ksq = fmaf(ak.z, ak.z, ksq); ksq = fmaf(ak.w, ak.w, ksq);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.x, bq.x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.z, bq.z, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.y, bq.y, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.w, bq.w, acc1, 0, 0, 0);
    }
  };
  // chunk c lives in ring slot c % kPrefetch until it is copied to the
  // wave's LDS buffer c & 1 (during chunk c - 1); the slot is then refilled
  // with chunk c + kPrefetch.  A wave's LDS operations complete in order, so
  // buffer c & 1 is rewritten only after chunk c - 2's reads of it.
  for (int c0 = 0; c0 < nchunks_p; c0 += kPrefetch) {
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
      const int c = c0 + i;
      mfma_chunk(c);
      stage_store(stg[(i + 1) % kPrefetch], c + 1);
      stage_load(stg[(i + 1) % kPrefetch], c + 1 + kPrefetch);
    }
  }
  __syncthreads();     // the score buffers below reuse every wave's staging slice
  ksq += xor_lane<16>(ksq);
  ksq += xor_lane<32>(ksq);
  // acc[r] = dim-share sum of K[key 4*quad + r of the tile] . Q[token row]
  const int ppitch = blk + 1;
  if (ndq == 1) {
    // one wave holds every dim: ordering keys go straight to LDS
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = quad * 4 + r;
      const double kn = __shfl(ksq, j, kWave);      // norm of tile key j sits in lane j
      const int gkey = kb * blk + kt * 16 + j;
      float o = __builtin_inff();
      if (gkey < a.n && t0 + row < a.T) {
        const double dot = (double)acc0[r] + (double)acc1[r];
        o = order_key(a.mode == 0 ? (float)(kn - 2.0 * dot) : (float)(-dot));
      }
      sc[row * ppitch + kt * 16 + j] = o;
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      part[(dq * kTokTile + row) * ppitch + kt * 16 + quad * 4 + r] = acc0[r] + acc1[r];
    if (lane < 16) knp[dq * blk + kt * 16 + lane] = ksq;
    __syncthreads();

    // combine dim shares -> ordering keys (thread <-> (token, key))
    float oval[kMaxBlk * kTokTile / (kScoreWaves * kWave)];
    const int nent = kTokTile * blk;
#pragma unroll
    for (int i = 0; i < kMaxBlk * kTokTile / (kScoreWaves * kWave); ++i) {
      const int e = tid + i * kScoreWaves * kWave;
      float o = __builtin_inff();
      if (e < nent) {
        const int tok = e / blk, kk = e - tok * blk;
        const int gkey = kb * blk + kk;
        if (gkey < a.n && t0 + tok < a.T) {
          double dot = 0.0, kn = 0.0;
          for (int s = 0; s < ndq; ++s) {
            dot += (double)part[(s * kTokTile + tok) * ppitch + kk];
            kn += knp[s * blk + kk];
          }
          o = order_key(a.mode == 0 ? (float)(kn - 2.0 * dot) : (float)(-dot));
        }
      }
      oval[i] = o;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxBlk * kTokTile / (kScoreWaves * kWave); ++i) {
      const int e = tid + i * kScoreWaves * kWave;
      if (e < nent) {
        const int tok = e / blk, kk = e - tok * blk;
        sc[tok * ppitch + kk] = oval[i];
      }
    }
    __syncthreads();
  }

  // ---- addressing loss: every ordering key of the tile goes to the
  // workspace (the softmax over all sub-keys needs them, not only the best k)
  if (a.addr_s) {
    float* dst = a.addr_s + ((int64_t)(u * 2 + h) * a.T + t0) * a.addr_np + kb * blk;
    for (int e = tid; e < kTokTile * blk; e += kScoreWaves * kWave) {
      const int r = e / blk, c = e - r * blk;
      if (t0 + r < a.T && kb * blk + c < a.n) dst[(int64_t)r * a.addr_np + c] = sc[r * ppitch + c];
    }
  }

  // ---- per token (wave w <-> token w): the k best of the block
  const int tw = t0 + wave;
  if (tw >= a.T) return;
  const int k = a.k;
  const float* srow = sc + wave * ppitch;
  auto cand = [&](int c) -> skey {
    const int gkey = kb * blk + c;
    return gkey < a.n ? pack_key(srow[c], gkey) : kEmptyKey;
  };
  skey x = cand(lane);
  sort_keys<64>(x);                               // the first 64, best first
  if (blk > kWave) {
    const skey th = readlane_k(x, k - 1);         // k-th best so far
    skey* sv = surv + wave * blk;
    int nsurv = 0;
    for (int c0 = kWave; c0 < blk; c0 += kWave) {
      const skey cx = cand(c0 + lane);
      const bool pass = cx < th;
      const unsigned long long m = __ballot(pass);
      if (pass) sv[nsurv + __popcll(m & ((1ull << lane) - 1ull))] = cx;
      nsurv += __popcll(m);
    }
    // the k best stay in lanes 0..k-1; survivors fill lanes k.. in batches,
    // and only the lane group that holds them is sorted
    const int fresh = kWave - k;
    for (int pos = 0; pos < nsurv; pos += fresh) {
      if (lane >= k) {
        const int c = pos + lane - k;
        x = c < nsurv ? sv[c] : kEmptyKey;
      }
      const int cnt = k + min(fresh, nsurv - pos);
      if (cnt <= 16) sort_keys<16>(x);
      else if (cnt <= 32) sort_keys<32>(x);
      else sort_keys<64>(x);
    }
  }
  if (lane < k) {
    const int64_t base = ((((int64_t)u * a.T + tw) * 2 + h) * a.nblk + kb) * k;
    a.half_o[base + lane] = key_value(x);
    a.half_i[base + lane] = key_index(x);
  }
}

int score_key_block(int units, int tokens, int n) {
  const int ntt = (tokens + kTokTile - 1) / kTokTile;
  int blk = kMaxBlk;
  while (blk > 64 && (int64_t)units * 2 * ntt * ((n + blk - 1) / blk) < 256) blk /= 2;
  return blk;
}

template <int kDimChunk, int kPrefetch>
size_t ka_smem_bytes(int half, int blk) {
  constexpr int kKPitch = kDimChunk + 4;
  const int ndq = kScoreWaves / (blk / 16);
  // dim-share partials / scores and the filter survivors reuse the two key
  // staging buffers once the contraction is done
  static_assert(sizeof(float) * 4 * kTokTile * (64 + 1) <= sizeof(float) * kStageRows * kKPitch, "partials");
  static_assert(sizeof(skey) * kTokTile * kMaxBlk <= sizeof(float) * kStageRows * kKPitch, "survivors");
  return sizeof(float) * kTokTile * (ka_query_width<kDimChunk, kPrefetch>(half, blk) + 4)   // queries
         + 2 * sizeof(float) * kStageRows * kKPitch                  // staged keys (double buffer)
         + sizeof(double) * ndq * blk;                               // key-norm partials
}

int ka_grid(const ChunkArgs& a) {
  const int ntt = (a.T + kTokTile - 1) / kTokTile;
  const int total = a.U * 2 * a.nblk * ntt;
  return 8 * ((total + 7) / 8);
}

namespace {

constexpr size_t kLdsBytes = 160 * 1024;

template <int DC, int PF, bool kFull>
hipError_t launch_ka_full(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ka_score_topk<DC, PF, kFull>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  return fw_launch(ka_score_topk<DC, PF, kFull>, dim3(ka_grid(a)), dim3(kScoreWaves * kWave),
                   (uint32_t)ka_smem_bytes<DC, PF>(a.half, a.key_block), s, tm, a);
}

template <int DC, int PF>
hipError_t launch_ka_as(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  // the kernel's own share / chunk arithmetic, on the host
  const int ndq = kScoreWaves / (a.key_block / 16);
  const int share = ((a.half + 16 * ndq - 1) / (16 * ndq)) * 16;
  const int nchunks = (share + DC - 1) / DC;
  const bool full = share % DC == 0 && ndq * share <= a.half && ka_chunks<DC, PF>(a.half, a.key_block) == nchunks;
  return full ? launch_ka_full<DC, PF, true>(a, s, tm) : launch_ka_full<DC, PF, false>(a, s, tm);
}

}  // namespace

hipError_t launch_ka(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  // wider chunks halve the barriers per contraction; they fit for d_h <= 256.
  // A ring deeper than the chunk count would only multiply zeros.
  if (ka_smem_bytes<64, 2>(a.half, a.key_block) <= kLdsBytes) {
    if (ka_chunks<64, 1>(a.half, a.key_block) == 1) return launch_ka_as<64, 1>(a, s, tm);
    return launch_ka_as<64, 2>(a, s, tm);
  }
  return launch_ka_as<32, 4>(a, s, tm);
}

}  // namespace fwpkm
