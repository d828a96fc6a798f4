// KA: sub-key scoring on the matrix cores, with the per-half top-k fused in.
//
// For every unit, query half h, token t and sub-key i this computes an
// ordering key o_h[t, i] whose ascending order is best-first:
//   IDW  o = ||K_h[i]||^2 - 2 q_h[t].K_h[i]   (= ||q_h - K_h[i]||^2 - ||q_h||^2)
//   dot  o = -(q_h[t].K_h[i])
// and keeps, per 256-key block, the k best (o asc, index asc).  The query's
// own norm ||q_h||^2 is common to every candidate of a half, so it is kept
// apart (qnorm) and added back only for the weights.
// [gist.science "Fast-weight Product Key Memory", section 2: sub-key
// codebooks K(1), K(2) scored in O(sqrt N), IDW score -log(eps+||q-K||^2);
// agifrontier tutorial, Product Key addressing: query split in two halves]
//
// The q.K contraction is a dense [keys x d_h] x [d_h x tokens] product per
// unit and half: it runs on v_mfma_f32_16x16x4_f32 with the query tile staged
// in LDS.  Every 32 dims the fp32 MFMA partial sums are folded into fp64
// accumulators and the key norms are summed in fp64, so the ordering keys
// carry far less rounding than the 1e-6 relative gap at which two candidates
// count as tied.
//
// Workgroup = 4 waves = one (unit, half, 256-key block, 16-token tile); wave w
// scores keys [w*64, w*64+64) of the block as four 16-key MFMA tiles.  Work
// items are laid out so that the token tiles sharing one key block run on one
// XCD (workgroup i is dispatched to XCD i % 8), which keeps the block's keys
// in that XCD's L2.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void ka_score_topk(ChunkArgs a) {
  extern __shared__ float smem[];
  const int half = a.half;
  const int qpitch = half + 4;
  float* qs = smem;                             // [16][qpitch]
  float* sc = smem + kTokTile * qpitch;         // [16][kKeyBlock + 4]
  constexpr int spitch = kKeyBlock + 4;

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

  // ---- stage the 16-token query tile (this half) in LDS
  const int half4 = half >> 2;
  for (int e = tid; e < kTokTile * half4; e += 256) {
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

  // ---- query norms (fp64 sums), once per token and half
  if (kb == 0) {
    for (int r = wave * 4; r < wave * 4 + 4; ++r) {
      const int t = t0 + r;
      double s = 0.0;
      for (int d = lane; d < half; d += kWave) {
        const double x = qs[r * qpitch + d];
        s += x * x;
      }
      s = wave_sum_d(s);
      if (lane == 0 && t < a.T) a.qnorm[((int64_t)u * a.T + t) * 2 + h] = (float)s;
    }
  }

  // ---- scores of 16 tokens x 64 keys per wave on the matrix cores
  const float* K = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + (int64_t)hh * a.n * half;
  const int key_base = kb * kKeyBlock + wave * 64;
  const int row = lane & 15;     // A row (key within tile) / B column (token)
  const int quad = lane >> 4;    // which 4-dim group of each 16-dim step
  const bool any_key = key_base < a.n;

  v4f acc[4];
  double acc64[4][4];
  double ksq[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    acc[kt] = v4f{0.f, 0.f, 0.f, 0.f};
    ksq[kt] = 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc64[kt][r] = 0.0;
  }
  if (any_key) {
    const float* krow[4];
    bool kvalid[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = key_base + kt * 16 + row;
      kvalid[kt] = key < a.n;
      krow[kt] = K + (int64_t)(kvalid[kt] ? key : 0) * half;
    }
    int steps = 0;
    for (int d0 = 0; d0 < half; d0 += 16) {
      const int d = d0 + quad * 4;
      const bool dvalid = d < half;
      float4 bq = make_float4(0.f, 0.f, 0.f, 0.f);
      if (dvalid) bq = *reinterpret_cast<const float4*>(&qs[row * qpitch + d]);
      float4 ak[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        ak[kt] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (dvalid && kvalid[kt]) ak[kt] = *reinterpret_cast<const float4*>(krow[kt] + d);
        ksq[kt] += (double)ak[kt].x * ak[kt].x + (double)ak[kt].y * ak[kt].y +
                   (double)ak[kt].z * ak[kt].z + (double)ak[kt].w * ak[kt].w;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[kt].x, bq.x, acc[kt], 0, 0, 0);
        acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[kt].y, bq.y, acc[kt], 0, 0, 0);
        acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[kt].z, bq.z, acc[kt], 0, 0, 0);
        acc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[kt].w, bq.w, acc[kt], 0, 0, 0);
      }
      if (++steps == 2) {  // fold every 32 dims into fp64
        steps = 0;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc64[kt][r] += (double)acc[kt][r];
          acc[kt] = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[kt][r] += (double)acc[kt][r];
    }
  }

  // ---- epilogue: ordering keys into LDS.  Lane holds keys 4*quad + r of each
  // tile for token `row`; the key norm of tile-key j sits in lanes j, j+16, ...
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    double kn = ksq[kt];
    kn += __shfl_xor(kn, 16, kWave);
    kn += __shfl_xor(kn, 32, kWave);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = quad * 4 + r;                 // key within the tile
      const double knj = __shfl(kn, j, kWave);
      const int key = key_base + kt * 16 + j;
      const int t = t0 + row;
      float o;
      if (key < a.n && t < a.T) {
        const double dot = acc64[kt][r];
        o = (a.mode == 0) ? (float)(knj - 2.0 * dot) : (float)(-dot);
        o = order_key(o);
      } else {
        o = __builtin_inff();
      }
      sc[row * spitch + wave * 64 + kt * 16 + j] = o;
    }
  }
  __syncthreads();

  // ---- per token: the k best of the block's 256 keys (k rounds of argmin)
  for (int r = wave * 4; r < wave * 4 + 4; ++r) {
    const int t = t0 + r;
    if (t >= a.T) break;
    float cv[4];
    int ci[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int local = lane + 64 * j;
      const int key = kb * kKeyBlock + local;
      cv[j] = sc[r * spitch + local];
      ci[j] = key < a.n ? key : kNoIndex;
      if (ci[j] == kNoIndex) cv[j] = __builtin_inff();
    }
    float mine_v;
    int mine_i;
    wave_select_k<4>(cv, ci, a.k, mine_v, mine_i);
    if (lane < a.k) {
      const int64_t base = ((((int64_t)u * a.T + t) * 2 + h) * a.nblk + kb) * a.k;
      a.half_o[base + lane] = mine_v;
      a.half_i[base + lane] = mine_i;
    }
  }
}

size_t ka_smem_bytes(int half) {
  return sizeof(float) * (size_t)kTokTile * ((half + 4) + (kKeyBlock + 4));
}

int ka_grid(const ChunkArgs& a) {
  const int ntt = (a.T + kTokTile - 1) / kTokTile;
  const int total = a.U * 2 * a.nblk * ntt;
  return 8 * ((total + 7) / 8);
}

hipError_t launch_ka(const ChunkArgs& a, hipStream_t s) {
  const size_t smem = ka_smem_bytes(a.half);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ka_score_topk), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)ka_smem_bytes(FWPKM_MAX_HALF_DIM));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(ka_score_topk, dim3(ka_grid(a)), dim3(256), smem, s, a);
  return hipGetLastError();
}

}  // namespace fwpkm
