// KD: per-row mean gradient and in-place SGD step on the touched V, K1 and
// K2 rows.
//
// For a row r touched by the n_r tokens of its segment (pairs in ascending
// token order):
//   V row   theta_r <- theta_r - lr * (1/n_r) sum_p w_p g_{t_p}
//   K1 row  IDW: theta_r <- theta_r - lr * (1/n_r) sum_p c_p (q1_{t_p} - theta_r)
//           dot: theta_r <- theta_r - lr * (1/n_r) sum_p c_p q1_{t_p}
//   K2 row  likewise with q2.
// All gradients are taken at the chunk's starting weights: each row is
// written once, by the wave that finishes it, after every wave that reads its
// old value has done so (within the workgroup), so updating in place is
// exact.
// [agifrontier tutorial "Fast-weight Product Key Memory", update equation
// theta' = theta - eta grad L_MSE; gist.science summary, section 2: Key and
// Value matrices updated online, gradients of a slot used several times in a
// chunk averaged; sciencestack.ai contents: no gradient clipping]
//
// Work distribution, over every list and unit of the chunk: a task is either
// one long segment (more than kShortSeg pairs), which the four waves of a
// workgroup split into contiguous quarters and combine in LDS in wave order,
// or up to four short segments, one per wave.  Every sum runs in a fixed
// order, so results do not depend on scheduling, and no atomics are used.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

// pref[i] = tasks of lists [0, i) for i in [0, L]; all threads of the block.
__device__ void task_prefix(const int* kinds, int L, int* pref, int* wtot) {
  constexpr int NT = kUpdWaves * kWave;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int per = (L + NT - 1) / NT;
  const int beg = tid * per;
  auto tasks = [&](int i) { return kinds[2 * i] + (kinds[2 * i + 1] + kUpdWaves - 1) / kUpdWaves; };
  int local = 0;
  for (int j = 0; j < per; ++j)
    if (beg + j < L) local += tasks(beg + j);
  int incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  int run = base + incl - local;
  for (int j = 0; j < per; ++j) {
    if (beg + j < L) {
      pref[beg + j] = run;
      run += tasks(beg + j);
    }
  }
  if (tid == NT - 1) pref[L] = run;
  __syncthreads();
}

// One wave's sum over sorted pairs [r0, r1) of a V list:  sum_p w_p g_{t_p}.
template <int R>
__device__ __forceinline__ void sum_value_pairs(const ChunkArgs& a, int u, const int* sorted,
                                                int r0, int r1, float4 (&acc)[R]) {
  const int lane = lane_id();
  const int width4 = a.dv >> 2;
  const float* sw = a.sel_w + (int64_t)u * a.P;
  const float* gbase = a.g + (int64_t)u * a.T * a.dv;
  for (int base = r0; base < r1; base += kWave) {
    const int nb = min(kWave, r1 - base);
    const int pl = lane < nb ? sorted[base + lane] : 0;
    const int tl = pl / a.k;
    const float wl = lane < nb ? sw[pl] : 0.f;
    for (int i = 0; i < nb; i += 8) {
      float4 gv[8][R];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int t = readlane_i(tl, min(i + jj, nb - 1));
        const float4* gr = reinterpret_cast<const float4*>(gbase + (int64_t)t * a.dv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = lane + 64 * r;
          gv[jj][r] = (i + jj < nb && c < width4) ? gr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (i + jj < nb) {
          const float w = readlane_f(wl, i + jj);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            acc[r].x += w * gv[jj][r].x; acc[r].y += w * gv[jj][r].y;
            acc[r].z += w * gv[jj][r].z; acc[r].w += w * gv[jj][r].w;
          }
        }
      }
    }
  }
}

// One wave's sum over sorted pairs [r0, r1) of a K list (half h):
//   IDW sum_p c_p (q_h[t_p] - old),  dot sum_p c_p q_h[t_p].
template <int R>
__device__ __forceinline__ void sum_key_pairs(const ChunkArgs& a, int u, int h, const int* sorted,
                                              int r0, int r1, const float4 (&old)[R],
                                              float4 (&acc)[R]) {
  const int lane = lane_id();
  const int width4 = a.half >> 2;
  const int b = u / a.H, hh = u - b * a.H;
  const float* cf = a.coef + (int64_t)h * a.U * a.P + (int64_t)u * a.P;
  const bool idw = a.mode == 0;
  for (int base = r0; base < r1; base += kWave) {
    const int nb = min(kWave, r1 - base);
    const int pl = lane < nb ? sorted[base + lane] : 0;
    const int tl = pl / a.k;
    const float cl = lane < nb ? cf[pl] : 0.f;
    for (int i = 0; i < nb; i += 8) {
      float4 qv[8][R];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int t = readlane_i(tl, min(i + jj, nb - 1));
        const float4* qr = reinterpret_cast<const float4*>(
            a.q + ((int64_t)(b * a.T + t) * a.H + hh) * a.dqk + h * a.half);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = lane + 64 * r;
          qv[jj][r] = (i + jj < nb && c < width4) ? qr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (i + jj < nb) {
          const float cc = readlane_f(cl, i + jj);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float4 x = qv[jj][r];
            if (idw) { x.x -= old[r].x; x.y -= old[r].y; x.z -= old[r].z; x.w -= old[r].w; }
            acc[r].x += cc * x.x; acc[r].y += cc * x.y; acc[r].z += cc * x.z; acc[r].w += cc * x.w;
          }
        }
      }
    }
  }
}

}  // namespace

template <int R>
__global__ __launch_bounds__(kUpdWaves * kWave) void kd_update(ChunkArgs a) {
  __shared__ int pref[kUpdMaxLists + 1];
  __shared__ int wtot[kUpdWaves];
  __shared__ float4 parts[kUpdWaves][kWave * R];
  const int L = 3 * a.U;
  task_prefix(a.seg_kinds, L, pref, wtot);
  const int total = pref[L];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int P = a.P;
  const float lr = a.lr;
  const int64_t UP = (int64_t)a.U * P;

  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    // (list, unit) holding this task
    int lo = 0, hi = L;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pref[mid] <= task) lo = mid; else hi = mid;
    }
    const int lu = lo;
    const int j = task - pref[lu];
    const int list = lu / a.U;
    const int u = lu - list * a.U;
    const int b = u / a.H, hh = u - b * a.H;
    const int64_t off = list * UP + (int64_t)u * P;                  // [3, U, P] arrays
    const int* sorted = a.sorted + off;
    const int* seg = a.seg_start + list * (UP + a.U) + (int64_t)u * (P + 1);
    const int n_long = a.seg_kinds[2 * lu];
    const bool is_long = j < n_long;
    int s;
    if (is_long) {
      s = a.long_seg[off + j];
    } else {
      const int si = (j - n_long) * kUpdWaves + wave;
      if (si >= a.seg_kinds[2 * lu + 1]) continue;                  // no wave-level barrier below
      s = a.short_seg[off + si];
    }
    const int s0 = seg[s], s1 = seg[s + 1];
    const int cnt = s1 - s0;
    int r0 = s0, r1 = s1;
    if (is_long) {
      const int ql = (cnt + kUpdWaves - 1) / kUpdWaves;
      r0 = min(s1, s0 + wave * ql);
      r1 = min(s1, r0 + ql);
    }
    const int row = a.keys[off + sorted[s0]];
    const bool finisher = !is_long || wave == 0;

    float4* trow;
    int width4;
    float4 old[R], acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (list == 0) {
      width4 = a.dv >> 2;
      trow = reinterpret_cast<float4*>(
          a.v + (int64_t)b * a.stride_v + ((int64_t)hh * a.n * a.n + row) * a.dv);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        old[r] = (finisher && c < width4) ? trow[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      sum_value_pairs<R>(a, u, sorted, r0, r1, acc);
    } else {
      const int h = list - 1;
      width4 = a.half >> 2;
      trow = reinterpret_cast<float4*>(
          (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + ((int64_t)hh * a.n + row) * a.half);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        old[r] = c < width4 ? trow[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      sum_key_pairs<R>(a, u, h, sorted, r0, r1, old, acc);
    }

    if (is_long) {
      // combine the four quarters in wave order
#pragma unroll
      for (int r = 0; r < R; ++r) parts[wave][lane + 64 * r] = acc[r];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float4 x = parts[0][lane + 64 * r];
#pragma unroll
          for (int w = 1; w < kUpdWaves; ++w) {
            const float4 y = parts[w][lane + 64 * r];
            x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
          }
          acc[r] = x;
        }
      }
    }
    if (finisher) {
      const float inv = 1.0f / (float)cnt;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = lane + 64 * r;
        if (c < width4) {
          float4 x = old[r];
          x.x -= lr * (acc[r].x * inv); x.y -= lr * (acc[r].y * inv);
          x.z -= lr * (acc[r].z * inv); x.w -= lr * (acc[r].w * inv);
          trow[c] = x;
        }
      }
    }
    if (is_long) __syncthreads();   // parts[] is reused by the next task
  }
}

hipError_t launch_kd(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const int r = (a.pw / 4 + 63) / 64;
  int64_t most = (int64_t)3 * a.U * (a.P / kUpdWaves + 1);   // tasks cannot exceed this
  int64_t gx = most < 2048 ? most : 2048;
  dim3 grid((unsigned)gx);
  dim3 block(kUpdWaves * kWave);
  if (r <= 1) return fw_launch(kd_update<1>, grid, block, 0, s, tm, a);
  if (r <= 2) return fw_launch(kd_update<2>, grid, block, 0, s, tm, a);
  if (r <= 4) return fw_launch(kd_update<4>, grid, block, 0, s, tm, a);
  return fw_launch(kd_update<8>, grid, block, 0, s, tm, a);
}

}  // namespace fwpkm
