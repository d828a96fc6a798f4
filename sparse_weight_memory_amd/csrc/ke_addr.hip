// KE: marginal-entropy addressing loss on the sub-keys (only when the
// configuration's addr_weight lambda is non-zero).
//
// Per unit and half h [gist.science "Fast-weight Product Key Memory",
// section 2: an auxiliary negative-entropy loss on the key matrices keeps slot
// usage balanced across a chunk; sciencestack.ai contents: "Addressing
// Optimization", "Marginal entropy loss"]:
//   s[t, i]  the token's score of sub-key i (IDW -log(eps + d[t, i]), dot q.K)
//   P[t, :]  softmax over all n sub-keys;  p = (1/T) sum_t P[t, :]
//   L_addr   = lambda * sum_i p_i log p_i
//   dL/ds[t, j] = lambda/T * P[t, j] (l_j - sum_i P[t, i] l_i),  l = log p
//   dL/dK[j]    = sum_t dL/ds[t, j] * ds[t, j]/dK[j], with
//                 IDW 2 (q_t - K[j]) / (eps + d[t, j]),  dot q_t.
// The score kernel leaves every ordering key in addr_s; ke_stats turns them
// into the coefficients c[t, j] = dL/ds * (IDW: 2 / (eps + d)) in place;
// ke_grad contracts them with the queries on the matrix cores,
//   dK[j] = sum_t c[t, j] q_t  (- (sum_t c[t, j]) K[j] for IDW),
// at the chunk's starting keys; ke_apply subtracts lr * dK from every key row
// after the update kernel has taken the MSE step.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kStatThreads = 1024;
constexpr int kMaxTokens = 1024;     // chunk-size limit of the API
constexpr int kMaxSubKeys = 4096;    // sqrt_slots limit of the API
constexpr float kMinUsage = 1e-30f;  // floor of p before the log (p > 0 in exact arithmetic)

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, xor_lane<32>(x));
  x = fmaxf(x, xor_lane<16>(x));
  x = fmaxf(x, xor_lane<8>(x));
  x = fmaxf(x, xor_lane<4>(x));
  x = fmaxf(x, xor_lane<2>(x));
  x = fmaxf(x, xor_lane<1>(x));
  return x;
}

}  // namespace

// One workgroup per (unit, half).
__global__ __launch_bounds__(kStatThreads) void ke_stats(ChunkArgs a) {
  __shared__ float s_max[kMaxTokens];
  __shared__ float s_inv[kMaxTokens];    // 1 / softmax sum
  __shared__ float s_ell[kMaxSubKeys];   // log marginal usage
  const int uh = blockIdx.x;
  const int u = uh >> 1, h = uh & 1;
  const int T = a.T, n = a.n;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  constexpr int kWaves = kStatThreads / kWave;
  float* S = a.addr_s + (int64_t)uh * T * n;
  const bool idw = a.mode == 0;
  auto dist = [&](float o, int t) {   // squared distance from the ordering key
    const float d = a.qnorm[((int64_t)u * T + t) * 2 + h] + o;
    return d > 0.f ? d : 0.f;
  };
  auto score = [&](float o, int t) { return idw ? -logf(a.eps + dist(o, t)) : -o; };

  // per token: max score and softmax sum
  for (int t = wave; t < T; t += kWaves) {
    const float* row = S + (int64_t)t * n;
    float m = -__builtin_inff();
    for (int i = lane; i < n; i += kWave) m = fmaxf(m, score(row[i], t));
    m = wave_max(m);
    float z = 0.f;
    for (int i = lane; i < n; i += kWave) z += expf(score(row[i], t) - m);
    z = wave_sum(z);
    if (lane == 0) {
      s_max[t] = m;
      s_inv[t] = 1.0f / z;
    }
  }
  __syncthreads();
  // per sub-key: marginal usage and its log
  const float inv_T = 1.0f / (float)T;
  for (int i = tid; i < n; i += kStatThreads) {
    float p = 0.f;
    for (int t = 0; t < T; ++t) p += expf(score(S[(int64_t)t * n + i], t) - s_max[t]) * s_inv[t];
    s_ell[i] = logf(fmaxf(p * inv_T, kMinUsage));
  }
  __syncthreads();
  // per token: sum_i P l_i, then the coefficients in place
  const float lam_T = a.addr_weight * inv_T;
  for (int t = wave; t < T; t += kWaves) {
    float* row = S + (int64_t)t * n;
    const float m = s_max[t], zi = s_inv[t];
    float acc = 0.f;
    for (int i = lane; i < n; i += kWave) acc += expf(score(row[i], t) - m) * zi * s_ell[i];
    const float pl = wave_sum(acc);
    for (int i = lane; i < n; i += kWave) {
      const float o = row[i];
      const float P = expf(score(o, t) - m) * zi;
      float c = lam_T * P * (s_ell[i] - pl);
      if (idw) c *= 2.0f / (a.eps + dist(o, t));
      row[i] = c;
    }
  }
}

namespace {

constexpr int kGradWaves = 16;
constexpr int kGradTile = 64;     // keys and dims of one workgroup's output block
constexpr int kTokChunk = 32;     // tokens staged in LDS at a time
constexpr int kGradPitch = kGradTile + 4;

}  // namespace

// dK for a 64-key x 64-dim block of one (unit, half); 16 waves, one 16x16
// output tile each.
__global__ __launch_bounds__(kGradWaves * kWave) void ke_grad(ChunkArgs a) {
  __shared__ float cs[kTokChunk][kGradPitch];   // coefficients [token][key]
  __shared__ float qs[kTokChunk][kGradPitch];   // queries [token][dim]
  const int uh = blockIdx.x;
  const int u = uh >> 1, h = uh & 1;
  const int b = u / a.H, hh = u - b * a.H;
  const int key0 = blockIdx.y * kGradTile, dim0 = blockIdx.z * kGradTile;
  const int T = a.T, n = a.n, half = a.half;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int kt = wave & 3, dt = wave >> 2;        // 16x16 tile of the block
  const int row = lane & 15, quad = lane >> 4;
  const float* S = a.addr_s + (int64_t)uh * T * n;
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  float csum = 0.f;                               // sum_t c[t, key0 + kt*16 + row] (lanes of quad 0..3)
  for (int t0 = 0; t0 < T; t0 += kTokChunk) {
    // stage: 2 * 32 * 64 floats, two per thread
    for (int e = tid; e < 2 * kTokChunk * kGradTile; e += kGradWaves * kWave) {
      const int which = e / (kTokChunk * kGradTile);
      const int r = (e / kGradTile) % kTokChunk, c = e % kGradTile;
      const int t = t0 + r;
      float x = 0.f;
      if (which == 0) {
        if (t < T && key0 + c < n) x = S[(int64_t)t * n + key0 + c];
        cs[r][c] = x;
      } else {
        if (t < T && dim0 + c < half)
          x = a.q[((int64_t)(b * T + t) * a.H + hh) * a.dqk + h * half + dim0 + c];
        qs[r][c] = x;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kTokChunk / 4; ++s) {
      const float av = cs[4 * s + quad][kt * 16 + row];   // A[key][token]
      const float bv = qs[4 * s + quad][dt * 16 + row];   // B[token][dim]
      csum += av;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // coefficient sums per key: lanes row, row+16, row+32, row+48 hold parts
  csum += xor_lane<16>(csum);
  csum += xor_lane<32>(csum);
  const bool idw = a.mode == 0;
  const float* Kt = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + (int64_t)hh * n * half;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kl = 4 * quad + r;                  // key of this accumulator inside the tile
    const float ck = __shfl(csum, kl, kWave);
    const int key = key0 + kt * 16 + kl, dim = dim0 + dt * 16 + row;
    if (key < n && dim < half) {
      float g = acc[r];
      if (idw) g -= ck * Kt[(int64_t)key * half + dim];
      a.addr_dk[((int64_t)uh * n + key) * half + dim] = g;
    }
  }
}

// K -= lr * dK for every key row of every unit and half.
__global__ __launch_bounds__(256) void ke_apply(ChunkArgs a) {
  const int64_t per = (int64_t)a.n * a.half;
  const int64_t total = (int64_t)a.U * 2 * per;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t uh = e / per, r = e - uh * per;
    const int u = (int)(uh >> 1), h = (int)(uh & 1);
    const int b = u / a.H, hh = u - b * a.H;
    float* K = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + (int64_t)hh * per;
    K[r] -= a.lr * a.addr_dk[e];
  }
}

hipError_t launch_ke_stats(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  return fw_launch(ke_stats, dim3(2 * a.U), dim3(kStatThreads), 0, s, tm, a);
}

hipError_t launch_ke_grad(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const dim3 grid(2 * a.U, (a.n + kGradTile - 1) / kGradTile, (a.half + kGradTile - 1) / kGradTile);
  return fw_launch(ke_grad, grid, dim3(kGradWaves * kWave), 0, s, tm, a);
}

hipError_t launch_ke_apply(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const int64_t total = (int64_t)a.U * 2 * a.n * a.half;
  const int64_t blocks = (total + 255) / 256;
  return fw_launch(ke_apply, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, tm, a);
}

}  // namespace fwpkm
