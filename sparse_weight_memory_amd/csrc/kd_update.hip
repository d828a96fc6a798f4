// KD: per-row mean gradient and in-place SGD step on the touched V, K1 and
// K2 rows, one wave per segment of the sorted pair lists.
//
// For a row r touched by the n_r tokens of its segment (pairs in ascending
// token order):
//   V row   theta_r <- theta_r - lr * (1/n_r) sum_p w_p g_{t_p}
//   K1 row  IDW: theta_r <- theta_r - lr * (1/n_r) sum_p c_p (q1_{t_p} - theta_r)
//           dot: theta_r <- theta_r - lr * (1/n_r) sum_p c_p q1_{t_p}
//   K2 row  likewise with q2.
// All gradients are taken at the chunk's starting weights: every row is owned
// by exactly one segment and reads only its own old value, so updating in
// place is exact.
// [agifrontier tutorial "Fast-weight Product Key Memory", update equation
// theta' = theta - eta grad L_MSE; gist.science summary, section 2: Key and
// Value matrices updated online, gradients of a slot used several times in a
// chunk averaged; sciencestack.ai contents: no gradient clipping]

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

template <int R>
__global__ __launch_bounds__(kUpdWaves * kWave) void kd_update(ChunkArgs a) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int lu = blockIdx.y;            // list * U + unit
  const int list = lu / a.U;
  const int u = lu - list * a.U;
  const int b = u / a.H, hh = u % a.H;
  const int P = a.P;
  const int64_t UP = (int64_t)a.U * P;
  const int nseg = a.nseg[lu];
  const int* sorted = a.sorted + list * UP + (int64_t)u * P;
  const int* seg = a.seg_start + list * (UP + a.U) + (int64_t)u * (P + 1);
  const int* keys = a.keys + list * UP + (int64_t)u * P;
  const float lr = a.lr;
  const int k = a.k;

  for (int j = blockIdx.x * kUpdWaves + wave; j < nseg; j += gridDim.x * kUpdWaves) {
    const int s0 = seg[j], s1 = seg[j + 1];
    const int cnt = s1 - s0;
    const int row = keys[sorted[s0]];
    if (list == 0) {
      // value row
      const int dv4 = a.dv >> 2;
      float4* vrow = reinterpret_cast<float4*>(
          a.v + (int64_t)b * a.stride_v + ((int64_t)hh * a.n * a.n + row) * a.dv);
      const float* sw = a.sel_w + (int64_t)u * P;
      float4 acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = s0; i < s1; ++i) {
        const int p = sorted[i];
        const int t = p / k;
        const float w = sw[p];
        const float4* gr = reinterpret_cast<const float4*>(a.g + ((int64_t)u * a.T + t) * a.dv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = lane + 64 * r;
          if (c < dv4) {
            const float4 gg = gr[c];
            acc[r].x += w * gg.x; acc[r].y += w * gg.y; acc[r].z += w * gg.z; acc[r].w += w * gg.w;
          }
        }
      }
      const float inv = 1.0f / (float)cnt;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        if (c < dv4) {
          float4 x = vrow[c];
          x.x -= lr * (acc[r].x * inv); x.y -= lr * (acc[r].y * inv);
          x.z -= lr * (acc[r].z * inv); x.w -= lr * (acc[r].w * inv);
          vrow[c] = x;
        }
      }
    } else {
      // sub-key row of half (list - 1)
      const int h = list - 1;
      const int half4 = a.half >> 2;
      float4* krow = reinterpret_cast<float4*>(
          (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + ((int64_t)hh * a.n + row) * a.half);
      const float* cf = a.coef + h * UP + (int64_t)u * P;
      float4 old[R], acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        old[r] = c < half4 ? krow[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const bool idw = a.mode == 0;
      for (int i = s0; i < s1; ++i) {
        const int p = sorted[i];
        const int t = p / k;
        const float cc = cf[p];
        const float4* qr = reinterpret_cast<const float4*>(
            a.q + ((int64_t)(b * a.T + t) * a.H + hh) * a.dqk + h * a.half);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = lane + 64 * r;
          if (c < half4) {
            float4 qq = qr[c];
            if (idw) { qq.x -= old[r].x; qq.y -= old[r].y; qq.z -= old[r].z; qq.w -= old[r].w; }
            acc[r].x += cc * qq.x; acc[r].y += cc * qq.y; acc[r].z += cc * qq.z; acc[r].w += cc * qq.w;
          }
        }
      }
      const float inv = 1.0f / (float)cnt;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        if (c < half4) {
          float4 x = old[r];
          x.x -= lr * (acc[r].x * inv); x.y -= lr * (acc[r].y * inv);
          x.z -= lr * (acc[r].z * inv); x.w -= lr * (acc[r].w * inv);
          krow[c] = x;
        }
      }
    }
  }
}

hipError_t launch_kd(const ChunkArgs& a, hipStream_t s) {
  const int w4 = ((a.dv > a.half ? a.dv : a.half) >> 2);
  const int r = (w4 + 63) / 64;
  int gx = (a.P + kUpdWaves - 1) / kUpdWaves;
  if (gx > 64) gx = 64;
  dim3 grid(gx, 3 * a.U);
  dim3 block(kUpdWaves * kWave);
  if (r <= 1) hipLaunchKernelGGL(kd_update<1>, grid, block, 0, s, a);
  else if (r <= 2) hipLaunchKernelGGL(kd_update<2>, grid, block, 0, s, a);
  else if (r <= 4) hipLaunchKernelGGL(kd_update<4>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(kd_update<8>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace fwpkm
