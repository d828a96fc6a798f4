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
// Key norms are summed in fp64, so the ordering keys carry far less rounding
// than the 1e-6 relative gap at which two candidates count as tied.
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
constexpr int kStepGroup = 8;      // 16-dim steps whose key operands are loaded together

__global__ __launch_bounds__(kScoreWaves * kWave) void ka_score_topk(ChunkArgs a) {
  extern __shared__ float smem[];
  const int half = a.half;
  const int blk = a.key_block;             // 64, 128 or 256
  const int nkt = blk / 16;                // key tiles per block
  const int ndq = kScoreWaves / nkt;       // dim shares per key tile
  const int qpitch = half + 4;
  float* qs = smem;                                      // [16][qpitch]
  float* part = qs + kTokTile * qpitch;                  // [ndq][16][blk + 1]
  double* knp = reinterpret_cast<double*>(part + ndq * kTokTile * (blk + 1));  // [ndq][blk]
  float* sc = part;                                      // [16][blk + 1], reuses part[0]
  skey* surv = reinterpret_cast<skey*>(knp + ndq * blk);    // [16][blk] filter survivors

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

  // ---- this wave's key operands: wave (kt, dq) = key tile kt over dim share
  // dq.  The first step group is requested before anything else, so its
  // latency overlaps the query staging.  (Requesting more at once does not
  // pay: a wave-wide load here touches 16 key rows, and the compute unit's
  // load path, not latency, then sets the pace.)
  const int kt = wave % nkt;
  const int dq = wave / nkt;
  const int row = lane & 15;          // A row (key) / B column (token)
  const int quad = lane >> 4;         // 4-dim group inside a 16-dim step
  const int share = ((half + 16 * ndq - 1) / (16 * ndq)) * 16;   // dims per share
  const int d_lo = dq * share;
  const int steps = share / 16;
  const int key = kb * blk + kt * 16 + row;
  const bool kvalid = key < a.n;
  const float* krow = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k +
                      ((int64_t)hh * a.n + (kvalid ? key : 0)) * half;
  auto step_dim = [&](int st) { return d_lo + st * 16 + quad * 4; };   // this lane's first dim of step st
  auto load_group = [&](float4 (&dst)[kStepGroup], int s0) {
#pragma unroll
    for (int j = 0; j < kStepGroup; ++j) {
      const int d = step_dim(s0 + j);
      const bool ok = s0 + j < steps && d < half;
      dst[j] = (ok && kvalid) ? *reinterpret_cast<const float4*>(krow + d)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float4 ak0[kStepGroup], ak1[kStepGroup];
  load_group(ak0, 0);

  // ---- stage the 16-token query tile (this half) in LDS
  const int half4 = half >> 2;
  for (int e = tid; e < kTokTile * half4; e += kScoreWaves * kWave) {
    const int r = e / half4, c4 = e - r * half4;
    const int t = t0 + r;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < a.T) {
      const float* qrow = a.q + ((int64_t)(b * a.T + t) * a.H + hh) * a.dqk + h * half;
      x = reinterpret_cast<const float4*>(qrow)[c4];
    }
    *reinterpret_cast<float4*>(&qs[r * qpitch + c4 * 4]) = x;
  }
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
  // of each step); a group's key operands are requested just before it runs.
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  double ksq = 0.0;
  auto mfma_group = [&](const float4 (&ak)[kStepGroup], int s0) {
#pragma unroll
    for (int j = 0; j < kStepGroup; ++j) {
      const int d = step_dim(s0 + j);
      const bool ok = s0 + j < steps && d < half;
      const float4 bq = ok ? *reinterpret_cast<const float4*>(&qs[row * qpitch + d])
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      ksq += (double)ak[j].x * ak[j].x + (double)ak[j].y * ak[j].y +
             (double)ak[j].z * ak[j].z + (double)ak[j].w * ak[j].w;
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[j].x, bq.x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[j].z, bq.z, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[j].y, bq.y, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[j].w, bq.w, acc1, 0, 0, 0);
    }
  };
  for (int s0 = 0; s0 < steps; s0 += 2 * kStepGroup) {
    mfma_group(ak0, s0);
    if (s0 + kStepGroup < steps) {
      load_group(ak1, s0 + kStepGroup);
      mfma_group(ak1, s0 + kStepGroup);
    }
    if (s0 + 2 * kStepGroup < steps) load_group(ak0, s0 + 2 * kStepGroup);
  }
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

size_t ka_smem_bytes(int half, int blk) {
  const int ndq = kScoreWaves / (blk / 16);
  return sizeof(float) * kTokTile * (half + 4)                       // queries
         + sizeof(float) * ndq * kTokTile * (blk + 1)                // dim-share partials / scores
         + sizeof(double) * ndq * blk                                // key-norm partials
         + sizeof(skey) * kTokTile * blk;                            // filter survivors
}

int ka_grid(const ChunkArgs& a) {
  const int ntt = (a.T + kTokTile - 1) / kTokTile;
  const int total = a.U * 2 * a.nblk * ntt;
  return 8 * ((total + 7) / 8);
}

hipError_t launch_ka(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ka_score_topk), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)std::max(ka_smem_bytes(FWPKM_MAX_HALF_DIM, 64), ka_smem_bytes(FWPKM_MAX_HALF_DIM, kMaxBlk)));
  if (attr != hipSuccess) return attr;
  return fw_launch(ka_score_topk, dim3(ka_grid(a)), dim3(kScoreWaves * kWave),
                   (uint32_t)ka_smem_bytes(a.half, a.key_block), s, tm, a);
}

}  // namespace fwpkm
