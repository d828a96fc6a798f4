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
// Work distribution, over every region of every list and unit: a task is
// either one long segment (more than kShortSeg pairs), which the W waves of a
// workgroup split into contiguous pieces and combine in LDS in wave order,
// or up to W short segments, one per wave.  A segment's record (row, first
// pair, pairs) and its sorted pair indices come straight from the grouping
// kernel; a pair's coefficient is loaded beside its data row, so a wave
// reaches the data rows after two dependent loads.  Every sum runs in a fixed order, so results do not
// depend on scheduling, and no atomics are used.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {


// Regions in XCD-affine order (unit count a multiple of 8): position r =
// ((x * 3 + list) * (U / 8) + ul) * regions + rg holds region
// (list * U + x * (U / 8) + ul) * regions + rg, so the regions of the units
// XCD x runs (see unit_affine_item) are positions [x L / 8, (x + 1) L / 8).
// The identity otherwise.
__device__ __forceinline__ int region_at(int r, const ChunkArgs& a) {
  const int units = a.U;
  if (units % kXcds != 0) return r;
  const int upx = units / kXcds;
  const int rg = r & (a.regions - 1);           // regions is a power of two
  const int rest = r >> a.region_bits;
  const int lx = fast_div(rest, a.div_upx);     // x * 3 + list
  const int ul = rest - lx * upx;
  const int x = lx / 3, list = lx - 3 * x;
  return (((list * units + x * upx + ul) << a.region_bits) | rg);
}

// pref[i] = tasks of the regions at positions [r0, i) (region_at order) for
// i in [r0, r1]; nlong / nshort / offs receive those regions' counts, by
// position.  All threads of the block take part.
template <int W>
__device__ void task_prefix(const ChunkArgs& a, int r0, int r1, int* pref,
                            int* nlong, int* nshort, int* offs, int* wtot) {
  constexpr int NT = W * kWave;
  const int tid = threadIdx.x, wave = tid / kWave;
  const int per = (r1 - r0 + NT - 1) / NT;
  const int beg = r0 + tid * per;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    if (beg + j < r1) {
      const int4 kd = a.kinds[region_at(beg + j, a)];
      nlong[beg + j] = kd.x;
      nshort[beg + j] = kd.y;
      offs[beg + j] = kd.z;
      local += kd.x + (kd.y + W - 1) / W;
    }
  }
  const int incl = wave_inclusive_scan(local);
  if (lane_id() == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  int run = base + incl - local;
  for (int j = 0; j < per; ++j) {
    if (beg + j < r1) {
      pref[beg + j] = run;
      run += nlong[beg + j] + (nshort[beg + j] + W - 1) / W;
    }
  }
  if (tid == NT - 1) pref[r1] = run;
  __syncthreads();
}

// The position in [r0, r1) of the region holding `task`: the largest r with
// pref[r] <= task (pref is nondecreasing and pref[r0] <= task < pref[r1]).
// A 64-way search per round: lane l tests position lo + l * step, and the
// lanes that pass are a prefix of the wave.
__device__ __forceinline__ int find_region(const int* pref, int r0, int r1, int task) {
  int lo = r0, span = r1 - r0;
  while (span > 1) {
    const int step = (span + kWave - 1) / kWave;
    const int at = lo + lane_id() * step;
    const bool ok = at < lo + span && pref[at] <= task;
    const int c = __popcll(__ballot(ok));        // >= 1: position lo passes
    lo += (c - 1) * step;
    span = min(step, r0 + (r1 - r0) - lo);
  }
  return lo;
}

// A table row as R float4 per lane, unguarded: columns past the row re-read
// its last float4.  Those lanes' sums are never stored, so the values need no
// mask, and nothing consumes the loads before the pair sums need them.
template <int R>
__device__ __forceinline__ void load_row(const float4* row, int width4, float4 (&out)[R]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = lane + 64 * r;
    out[r] = row[c < width4 ? c : width4 - 1];
  }
}

// Token of pair p = t*k + m without an integer divide: (p + 1/2) / k lies at
// least 1/(2k) >= 1/64 away from an integer, relative 2e-6 at p < 8192, far
// above the reciprocal's error.
__device__ __forceinline__ int token_of(int p, int k) {
  return (int)(((float)p + 0.5f) * __builtin_amdgcn_rcpf((float)k));
}

// One wave's sum over the sorted pairs pay[0, n) of a V segment:
// sum_p w_p g_{t_p}.  NB data rows are in flight at a time.  The row's
// current value goes into `old`, loaded in the first round beside the pairs'
// data (loads outstanding at a loop's head would be waited for there).
template <int R, int NB>
__device__ __forceinline__ void sum_value_pairs(const ChunkArgs& a, int u, const int* pay,
                                                int n, const float4* trow, int width4,
                                                float4 (&old)[R], float4 (&acc)[R]) {
  const int lane = lane_id();
  const float* gbase = a.g + (int64_t)u * a.T * a.dv;
  const float* sw = a.sel_w + (int64_t)u * a.P;
  for (int base = 0; base < n; base += kWave) {
    const int nb = min(kWave, n - base);
    const int pl = lane < nb ? pay[base + lane] : 0;
    const int tl = token_of(pl, a.k);
    float wl = 0.f;
    for (int i = 0; i < nb; i += NB) {
      float4 gv[NB][R];
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
        const int t = readlane_i(tl, min(i + jj, nb - 1));
        const float4* gr = reinterpret_cast<const float4*>(gbase + (int64_t)t * a.dv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = lane + 64 * r;
          gv[jj][r] = (i + jj < nb && c < width4) ? gr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      // the pairs' weights and the row's value go out behind the first
      // round's data rows (loads outstanding at a loop's head are waited for
      // there); lanes >= nb read pair 0's weight, never used
      if (i == 0) {
        wl = sw[pl];
        if (base == 0) load_row<R>(trow, width4, old);
      }
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
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

// One wave's sum over the pairs pay[0, n) of a K segment (half h):
//   IDW sum_p c_p (q_h[t_p] - old),  dot sum_p c_p q_h[t_p];
// `old` (the row's current value) is loaded as for value segments.
template <int R, int NB>
__device__ __forceinline__ void sum_key_pairs(const ChunkArgs& a, int u, int h, const int* pay,
                                              int n, const float4* trow, int width4,
                                              float4 (&old)[R], float4 (&acc)[R]) {
  const int lane = lane_id();
  const int b = fast_div(u, a.div_H), hh = u - b * a.H;
  const bool idw = a.mode == 0;
  const float* cf = a.coef + (int64_t)h * a.U * a.P + (int64_t)u * a.P;
  for (int base = 0; base < n; base += kWave) {
    const int nb = min(kWave, n - base);
    const int pl = lane < nb ? pay[base + lane] : 0;
    const int tl = token_of(pl, a.k);
    float cl = 0.f;
    for (int i = 0; i < nb; i += NB) {
      float4 qv[NB][R];
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
        const int t = readlane_i(tl, min(i + jj, nb - 1));
        const float4* qr = reinterpret_cast<const float4*>(
            a.q + ((int64_t)(b * a.T + t) * a.H + hh) * a.dqk + h * a.half);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = lane + 64 * r;
          qv[jj][r] = (i + jj < nb && c < width4) ? qr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      // coefficients and the row's value behind the first round's data rows
      if (i == 0) {
        cl = cf[pl];
        if (base == 0) load_row<R>(trow, width4, old);
      }
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
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

// Waves per SIMD each variant is compiled for: two workgroups of W waves per
// compute unit (four SIMDs), so a chunk's tasks fit on the device at once
// (the register budget per wave is 512 / waves).
template <int W>
constexpr int kd_waves_per_simd() { return 2 * W / 4; }
constexpr int kKdResidentPerCu = 2;

// LDS of one update workgroup for L regions: partial sums, then the region
// table.
template <int R, int W>
__host__ __device__ constexpr size_t kd_parts_bytes() {
  return sizeof(float4) * (size_t)W * kWave * R;
}

}  // namespace

template <int R, int W, int NB>
__global__ __launch_bounds__(W * kWave, kd_waves_per_simd<W>()) void kd_update(ChunkArgs a) {
  extern __shared__ float4 kd_lds[];
  float4* parts = kd_lds;                                             // [W][64 R]
  const int L = 3 * a.U * a.regions;
  int* pref = reinterpret_cast<int*>(kd_lds + (size_t)W * kWave * R); // [L + 1]
  int* nlong = pref + L + 1;                                          // [L]
  int* nshort = nlong + L;                                            // [L]
  int* offs = nshort + L;                                             // [L]
  int* wtot = offs + L;                                               // [W]
  // workgroups of XCD x take the tasks of that XCD's units (the grid is a
  // multiple of 8 then) and count only those regions; otherwise every
  // workgroup strides over all tasks
  int r_lo = 0, r_hi = L, t_first = blockIdx.x, t_step = gridDim.x;
  if (a.U % kXcds == 0) {
    r_lo = (blockIdx.x % kXcds) * (L / kXcds);
    r_hi = r_lo + L / kXcds;
    t_first = blockIdx.x / kXcds;
    t_step = gridDim.x / kXcds;
  }
  task_prefix<W>(a, r_lo, r_hi, pref, nlong, nshort, offs, wtot);
  const int t_end = pref[r_hi];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int P = a.P;
  const float lr = a.lr;

  for (int task = t_first; task < t_end; task += t_step) {
    const int lo = find_region(pref, r_lo, r_hi, task);   // region (position) holding this task
    const int j = task - pref[lo];
    const int lu = region_at(lo, a) >> a.region_bits;   // list * U + unit
    const int list = fast_div(lu, a.div_U);
    const int u = lu - list * a.U;
    const int b = fast_div(u, a.div_H), hh = u - b * a.H;
    const int64_t lbase = (int64_t)lu * P;
    const int nl = nlong[lo];
    const bool is_long = j < nl;
    int4 rec;
    if (is_long) {
      rec = a.long_rec[lbase + offs[lo] + j];
    } else {
      const int si = (j - nl) * W + wave;
      if (si >= nshort[lo]) continue;                              // no barrier on this path
      rec = a.short_rec[lbase + offs[lo] + si];
    }
    const int row = rec.x, cnt = rec.z;
    int p0 = rec.y, np = cnt;
    if (is_long) {
      const int ql = (cnt + W - 1) / W;
      const int r0 = min(cnt, wave * ql);
      np = min(cnt, r0 + ql) - r0;
      p0 += r0;
    }
    const int* pay = a.pay + lbase + p0;
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
      // every wave loads the row (used by the finisher only), beside the pairs
      if (np <= 0) load_row<R>(trow, width4, old);
      sum_value_pairs<R, NB>(a, u, pay, np, trow, width4, old, acc);
    } else {
      const int h = list - 1;
      width4 = a.half >> 2;
      trow = reinterpret_cast<float4*>(
          (h == 0 ? a.k1 : a.k2) + (int64_t)b * a.stride_k + ((int64_t)hh * a.n + row) * a.half);
      if (np <= 0) load_row<R>(trow, width4, old);
      sum_key_pairs<R, NB>(a, u, h, pay, np, trow, width4, old, acc);
    }

    if (is_long) {
      // combine the W pieces in wave order
#pragma unroll
      for (int r = 0; r < R; ++r) parts[wave * kWave * R + lane + 64 * r] = acc[r];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float4 x = parts[lane + 64 * r];
          for (int w = 1; w < W; ++w) {
            const float4 y = parts[w * kWave * R + lane + 64 * r];
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

namespace {

int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

template <int R, int W, int NB>
hipError_t launch_kd_as(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  const int64_t L = (int64_t)3 * a.U * a.regions;
  const size_t smem = kd_parts_bytes<R, W>() + sizeof(int) * (size_t)(4 * L + 1 + W);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&kd_update<R, W, NB>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(kd_parts_bytes<R, W>() + sizeof(int) * (size_t)(4 * kUpdMaxLists + 1 + W)));
  if (attr != hipSuccess) return attr;
  // tasks cannot exceed long segments + short groups of W, per region; more
  // workgroups than fit on the device at once would only queue behind the
  // first ones, so the grid stops at what is resident (tasks loop)
  const int64_t most = (int64_t)3 * a.U * a.P / (kShortSeg + 1) +
                       (int64_t)3 * a.U * a.P / W + L;
  const int64_t resident = (int64_t)kKdResidentPerCu * device_cus();
  int64_t gx = most < resident ? most : resident;
  if (a.U % kXcds == 0) gx = (gx + kXcds - 1) / kXcds * kXcds;   // whole rounds over the XCDs
  return fw_launch(kd_update<R, W, NB>, dim3((unsigned)gx), dim3(W * kWave), (uint32_t)smem, s, tm, a);
}

}  // namespace

hipError_t launch_kd(const ChunkArgs& args, hipStream_t s, const LaunchTiming* tm) {
  const ChunkArgs a = with_divisors(args);
  const int r = (a.pw / 4 + 63) / 64;
  // (float4 per lane per row, waves, rows in flight): the largest of each
  // that keeps two workgroups per compute unit without register spills
  if (r <= 1) return launch_kd_as<1, 16, 4>(a, s, tm);
  if (r <= 2) return launch_kd_as<2, 8, 8>(a, s, tm);
  if (r <= 4) return launch_kd_as<4, 4, 4>(a, s, tm);
  return launch_kd_as<8, 4, 2>(a, s, tm);
}

}  // namespace fwpkm
