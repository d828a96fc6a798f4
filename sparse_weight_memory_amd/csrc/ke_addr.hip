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
// The score kernel leaves every ordering key o in addr_s (IDW: the squared
// distance is qnorm + o; dot: the score is -o).  For IDW the softmax of
// -log(eps + d) is u / sum u with u = 1 / (eps + d), so no exp or log is taken
// there; dot scores take the usual max-shifted softmax.
//   ke_tokstats  per token: shift m (dot) and 1 / softmax sum
//   ke_usage     per sub-key: p = mean_t P[t, :] and l = log p, summed over
//                tokens in a fixed order (deterministic)
//   ke_coef      per token: sum_i P l_i, then c[t, j] = dL/ds * (IDW:
//                2 / (eps + d)) written over the scores in place
// ke_grad contracts c with the queries on the matrix cores,
//   dK[j] = sum_t c[t, j] q_t  (- (sum_t c[t, j]) K[j] for IDW),
// at the chunk's starting keys; ke_apply subtracts lr * dK from every key row
// after the update kernel has taken the MSE step.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kStatWaves = 16;       // one token (or 64 sub-keys) per wave
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

// One token's view of its score row: turns an ordering key into the
// unnormalised softmax term and the IDW factor 1 / (eps + d).  The score mode
// is a template argument so that no branch sits between a row's loads.
template <bool kIdw>
struct TokenRow {
  float eps, qn, m;
  __device__ __forceinline__ float inv_dist(float o) const {
    const float d = qn + o;
    return 1.0f / (eps + (d > 0.f ? d : 0.f));
  }
  // exp(s - m): IDW u = 1 / (eps + d) (m = 0), dot exp(-o - m)
  __device__ __forceinline__ float term(float o) const { return kIdw ? inv_dist(o) : expf(-o - m); }
};

template <bool kIdw>
__device__ __forceinline__ TokenRow<kIdw> token_row(const ChunkArgs& a, int u, int h, int t, float m) {
  TokenRow<kIdw> r;
  r.eps = a.eps;
  r.qn = kIdw ? a.qnorm[((int64_t)u * a.T + t) * 2 + h] : 0.f;
  r.m = m;
  return r;
}

}  // namespace

// Loads of a score row run kRowLoads at a time across the padded pitch (every
// load in range, none behind a branch); values past n are masked to zero in
// sums by AND-ing their bits, so no load is ever made conditional.
constexpr int kRowLoads = kAddrPad / kWave;
static_assert(kRowLoads * kWave == kAddrPad, "row pitch is a whole number of load batches");

// The mask goes through an empty asm so the compiler cannot rewrite the AND
// as a select and then move the load behind a branch (which would wait for
// every load on its own).
__device__ __forceinline__ float keep_if(float x, bool ok) {
  unsigned int m = ok ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return __uint_as_float(__float_as_uint(x) & m);
}

// Work item of a unit-major flat grid with `per_half` items per (unit, half):
// (unit * 2 + half, item within the half), XCD-affine (unit_affine_item).
struct HalfItem {
  int uh, i;
};
__device__ __forceinline__ HalfItem half_item(int units, int per_half) {
  const int item = unit_affine_item(blockIdx.x, units, 2 * per_half);
  const int uh = item / per_half;
  return {uh, item - uh * per_half};
}

// grid 2U * ceil(T / 16) (unit-major): one wave per token.
template <bool kIdw>
__global__ __launch_bounds__(kStatWaves * kWave) void ke_tokstats(ChunkArgs a) {
  const HalfItem it = half_item(a.U, (a.T + kStatWaves - 1) / kStatWaves);
  const int uh = it.uh, u = uh >> 1, h = uh & 1;
  const int t = it.i * kStatWaves + (int)(threadIdx.x / kWave);
  const int lane = lane_id(), n = a.n, np = a.addr_np;
  if (t >= a.T) return;
  const float* row = a.addr_s + ((int64_t)uh * a.T + t) * np;
  float m = 0.f;
  if (!kIdw) {                // dot: m = max_i s_i = max_i (-o_i); past n reread column n-1
    float hi = -__builtin_inff();
    for (int i0 = 0; i0 < np; i0 += kAddrPad) {
      float x[kRowLoads];
#pragma unroll
      for (int j = 0; j < kRowLoads; ++j) {
        const int i = i0 + j * kWave + lane;
        x[j] = row[i < n ? i : n - 1];
      }
#pragma unroll
      for (int j = 0; j < kRowLoads; ++j) hi = fmaxf(hi, -x[j]);
    }
    m = wave_max(hi);
  }
  const TokenRow<kIdw> tr = token_row<kIdw>(a, u, h, t, m);
  float z = 0.f;
  for (int i0 = 0; i0 < np; i0 += kAddrPad) {
    float x[kRowLoads];
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j) x[j] = row[i0 + j * kWave + lane];
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j) z += keep_if(tr.term(x[j]), i0 + j * kWave + lane < n);
  }
  z = wave_sum(z);
  if (lane == 0) {
    float* st = a.addr_tok + ((int64_t)uh * a.T + t) * 2;
    st[0] = m;
    st[1] = 1.0f / z;
  }
}

// grid 2U * ceil(n / 64) (unit-major): lane = sub-key, waves stride over
// tokens; the 16 partial sums of a sub-key are added in wave order.
template <bool kIdw>
__global__ __launch_bounds__(kStatWaves * kWave) void ke_usage(ChunkArgs a) {
  constexpr int kTokLoads = 8;            // tokens of one wave in flight
  __shared__ float part[kStatWaves][kWave];
  const HalfItem it = half_item(a.U, (a.n + kWave - 1) / kWave);
  const int uh = it.uh, u = uh >> 1, h = uh & 1;
  const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
  const int i = it.i * kWave + lane;                // < addr_np: the load is in range
  const int n = a.n, T = a.T, np = a.addr_np;
  const float* S = a.addr_s + (int64_t)uh * T * np;
  const float* st = a.addr_tok + (int64_t)uh * T * 2;
  float acc = 0.f;
  for (int t0 = wave; t0 < T; t0 += kStatWaves * kTokLoads) {
    float x[kTokLoads], zi[kTokLoads];
    TokenRow<kIdw> tr[kTokLoads];
#pragma unroll
    for (int j = 0; j < kTokLoads; ++j) {
      const int t = t0 + j * kStatWaves;
      const int tc = t < T ? t : T - 1;
      x[j] = S[(int64_t)tc * np + i];
      tr[j] = token_row<kIdw>(a, u, h, tc, kIdw ? 0.f : st[2 * tc]);
      zi[j] = st[2 * tc + 1];
    }
#pragma unroll
    for (int j = 0; j < kTokLoads; ++j)
      acc += keep_if(tr[j].term(x[j]) * zi[j], t0 + j * kStatWaves < T);
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && i < n) {
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < kStatWaves; ++w) p += part[w][lane];
    a.addr_ell[(int64_t)uh * n + i] = logf(fmaxf(p / (float)T, kMinUsage));
  }
}

// grid 2U * ceil(T / 16) (unit-major): one wave per token; scores become
// coefficients (pad columns receive values that no reader uses).
template <bool kIdw>
__global__ __launch_bounds__(kStatWaves * kWave) void ke_coef(ChunkArgs a) {
  const HalfItem it = half_item(a.U, (a.T + kStatWaves - 1) / kStatWaves);
  const int uh = it.uh, u = uh >> 1, h = uh & 1;
  const int t = it.i * kStatWaves + (int)(threadIdx.x / kWave);
  const int lane = lane_id(), n = a.n, np = a.addr_np;
  if (t >= a.T) return;
  float* row = a.addr_s + ((int64_t)uh * a.T + t) * np;
  const float* ell = a.addr_ell + (int64_t)uh * n;
  const float* st = a.addr_tok + ((int64_t)uh * a.T + t) * 2;
  const TokenRow<kIdw> tr = token_row<kIdw>(a, u, h, t, st[0]);
  const float zi = st[1];
  float acc = 0.f;
  for (int i0 = 0; i0 < np; i0 += kAddrPad) {
    float x[kRowLoads], l[kRowLoads];
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j) {
      const int i = i0 + j * kWave + lane;
      x[j] = row[i];
      l[j] = ell[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j)
      acc += keep_if(tr.term(x[j]) * zi * l[j], i0 + j * kWave + lane < n);
  }
  const float pl = wave_sum(acc);
  const float lam_T = a.addr_weight / (float)a.T;
  for (int i0 = 0; i0 < np; i0 += kAddrPad) {
    float x[kRowLoads], l[kRowLoads];
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j) {
      const int i = i0 + j * kWave + lane;
      x[j] = row[i];
      l[j] = ell[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < kRowLoads; ++j) {
      float c = lam_T * (tr.term(x[j]) * zi) * (l[j] - pl);
      if (kIdw) c *= 2.0f * tr.inv_dist(x[j]);
      row[i0 + j * kWave + lane] = c;
    }
  }
}

namespace {

constexpr int kGradWaves = 16;
constexpr int kGradTile = 64;     // keys and dims of one workgroup's output block
constexpr int kTokChunk = 64;     // tokens staged in LDS at a time
constexpr int kGradPitch = kGradTile + 4;
constexpr int kRowsPerPass = kGradWaves;                  // one staged row per wave per load
constexpr int kLoadsPerThread = 2 * kTokChunk / kRowsPerPass;   // coefficient and query rows

}  // namespace

// dK for a 64-key x 64-dim block of one (unit, half); 16 waves, one 16x16
// output tile each.  The next 64-token slice of coefficients and queries is
// loaded into registers while the current one feeds the matrix cores.
__global__ __launch_bounds__(kGradWaves * kWave) void ke_grad(ChunkArgs a) {
  __shared__ float cs[kTokChunk][kGradPitch];   // coefficients [token][key]
  __shared__ float qs[kTokChunk][kGradPitch];   // queries [token][dim]
  const int kty = (a.n + kGradTile - 1) / kGradTile, dtz = (a.half + kGradTile - 1) / kGradTile;
  const HalfItem it = half_item(a.U, kty * dtz);     // grid 2U * kty * dtz, unit-major
  const int uh = it.uh;
  const int u = uh >> 1, h = uh & 1;
  const int b = u / a.H, hh = u - b * a.H;
  const int ky = it.i / dtz;
  const int key0 = ky * kGradTile, dim0 = (it.i - ky * dtz) * kGradTile;
  const int T = a.T, n = a.n, half = a.half;
  const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
  const int kt = wave & 3, dt = wave >> 2;        // 16x16 tile of the block
  const int row = lane & 15, quad = lane >> 4;
  const int np = a.addr_np;
  const float* S = a.addr_s + (int64_t)uh * T * np;
  const float* Q = a.q + (int64_t)b * T * a.H * a.dqk + (int64_t)hh * a.dqk + h * half;
  const int64_t q_tok = (int64_t)a.H * a.dqk;     // query stride between tokens
  // this lane's column in the staged rows: key columns past n fall in the
  // row pitch's pad, dims past d_h are clamped; both are masked to zero
  const bool key_ok = key0 + lane < n, dim_ok = dim0 + lane < half;
  const int key_c = key0 + lane, dim_c = dim_ok ? dim0 + lane : half - 1;
  float pre[kLoadsPerThread];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < kLoadsPerThread; ++j) {
      const int r = wave + kRowsPerPass * (j % (kLoadsPerThread / 2));
      const int t = t0 + r;
      const int tc = t < T ? t : T - 1;
      pre[j] = j < kLoadsPerThread / 2 ? S[(int64_t)tc * np + key_c] : Q[tc * q_tok + dim_c];
    }
  };
  // the starting key rows of this lane's four outputs (IDW term), loaded
  // up front with clamped indices so that they land during the loop
  const bool idw = a.mode == 0;
  const float* Kt = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + (int64_t)hh * n * half;
  const int out_dim = dim0 + dt * 16 + row;
  float kv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = key0 + kt * 16 + 4 * quad + r;
    kv[r] = Kt[(int64_t)(key < n ? key : n - 1) * half + (out_dim < half ? out_dim : half - 1)];
  }
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  float csum = 0.f;                               // sum_t c[t, key0 + kt*16 + row] (lanes of quad 0..3)
  fetch(0);
  for (int t0 = 0; t0 < T; t0 += kTokChunk) {
#pragma unroll
    for (int j = 0; j < kLoadsPerThread; ++j) {
      // masked here, after the loads have landed: rows past T, key columns
      // in the pitch's pad and clamped dims stage as zero
      const int r = wave + kRowsPerPass * (j % (kLoadsPerThread / 2));
      if (j < kLoadsPerThread / 2) cs[r][lane] = keep_if(pre[j], t0 + r < T && key_ok);
      else qs[r][lane] = keep_if(pre[j], t0 + r < T && dim_ok);
    }
    __syncthreads();
    fetch(t0 + kTokChunk);                        // past the end: clamped, masked, unused
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
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kl = 4 * quad + r;                  // key of this accumulator inside the tile
    const float ck = __shfl(csum, kl, kWave);
    const int key = key0 + kt * 16 + kl;
    if (key < n && out_dim < half) {
      float g = acc[r];
      if (idw) g -= ck * kv[r];
      a.addr_dk[((int64_t)uh * n + key) * half + out_dim] = g;
    }
  }
}

// K -= lr * dK for every key row of every unit and half; grid U * bpu
// (unit-major): the bpu workgroups of a unit stride over its 2 n d_h entries.
__global__ __launch_bounds__(256) void ke_apply(ChunkArgs a, int bpu) {
  const int64_t per = (int64_t)a.n * a.half;
  const int item = unit_affine_item(blockIdx.x, a.U, bpu);
  const int unit = item / bpu, w = item - unit * bpu;
  const int64_t e_end = ((int64_t)unit + 1) * 2 * per;
  for (int64_t e = (int64_t)unit * 2 * per + (int64_t)w * blockDim.x + threadIdx.x; e < e_end;
       e += (int64_t)bpu * blockDim.x) {
    const int64_t uh = e / per, r = e - uh * per;
    const int u = (int)(uh >> 1), h = (int)(uh & 1);
    const int b = u / a.H, hh = u - b * a.H;
    float* K = (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + (int64_t)hh * per;
    K[r] -= a.lr * a.addr_dk[e];
  }
}

hipError_t launch_ke_stats(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  // one timed span: the first launch stamps the start, the last the end
  LaunchTiming first, last;
  if (tm) {
    first.beg = tm->beg;
    last.end = tm->end;
  }
  const dim3 tok_grid((unsigned)(2 * a.U * ((a.T + kStatWaves - 1) / kStatWaves)));   // unit-major
  const dim3 key_grid((unsigned)(2 * a.U * ((a.n + kWave - 1) / kWave)));
  const dim3 block(kStatWaves * kWave);
  const bool idw = a.mode == 0;
  hipError_t e = idw ? fw_launch(ke_tokstats<true>, tok_grid, block, 0, s, tm ? &first : nullptr, a)
                     : fw_launch(ke_tokstats<false>, tok_grid, block, 0, s, tm ? &first : nullptr, a);
  if (e == hipSuccess)
    e = idw ? fw_launch(ke_usage<true>, key_grid, block, 0, s, nullptr, a)
            : fw_launch(ke_usage<false>, key_grid, block, 0, s, nullptr, a);
  if (e == hipSuccess)
    e = idw ? fw_launch(ke_coef<true>, tok_grid, block, 0, s, tm ? &last : nullptr, a)
            : fw_launch(ke_coef<false>, tok_grid, block, 0, s, tm ? &last : nullptr, a);
  return e;
}

hipError_t launch_ke_grad(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const dim3 grid((unsigned)(2 * a.U * ((a.n + kGradTile - 1) / kGradTile) *
                             ((a.half + kGradTile - 1) / kGradTile)));   // unit-major
  return fw_launch(ke_grad, grid, dim3(kGradWaves * kWave), 0, s, tm, a);
}

hipError_t launch_ke_apply(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const int64_t per_unit = (int64_t)2 * a.n * a.half;
  int64_t bpu = (per_unit + 255) / 256;                 // workgroups per unit, about 4096 in all
  const int64_t cap = 4096 / a.U > 0 ? 4096 / a.U : 1;
  if (bpu > cap) bpu = cap;
  return fw_launch(ke_apply, dim3((unsigned)(a.U * bpu)), dim3(256), 0, s, tm, a, (int)bpu);
}

}  // namespace fwpkm
