// KB: Cartesian top-k, softmax weights, value gather-reduce and the
// fast-weight backward, one wave per (unit, token).
//
// Read [sciencestack.ai "Fast-weight Product Key Memory", contents entry
// "Top-k Key-value Memory"; gist.science summary, section 2]:
//   candidates (a, b) from the per-half best-k lists, ordering key
//   o1[a] + o2[b], slot a*n + b; keep the k best (key asc, slot asc).
//   IDW weights  w_m = u_m / sum u,  u_m = 1 / (eps + D_m),
//                D_m = ||q1||^2 + ||q2||^2 + o1 + o2  (= ||q - K_slot||^2),
//   which is softmax(-log(eps + D)) written without the log/exp pair;
//   dot weights  w = softmax(q.K_slot).
//   out_t = sum_m w_m V[slot_m], summed in rank order.
// Only candidates (i, j) with (i+1)(j+1) <= k can reach the top k (every
// (i', j') with i' <= i, j' <= j orders before them), so at most
// sum_i floor(k/i) <= 64 candidates (k <= 20) are ranked, one per lane.
//
// Backward of L = sum_t 1/2 ||out_t - y_t||^2 at the chunk's starting weights
// [agifrontier tutorial, update equation; sciencestack.ai contents: MSE loss,
// summation reduction, weighting gradient by row contribution]:
//   g_t = out_t - y_t,  dL/dV[slot_m] = w_m g_t (left implicit: (slot, pair)
//   and w are stored, the value gradient is formed in the update kernel),
//   delta_m = w_m (g_t.V[slot_m] - g_t.out_t),
//   IDW coefficient c_m = 2 delta_m u_m   (dL/dK1[a] = sum c_m (q1 - K1[a])),
//   dot coefficient c_m = delta_m         (dL/dK1[a] = sum c_m q1).
// Candidates of one token that share a K1 (K2) row are merged into one
// (row, token) pair here, so that the update divides by the number of
// tokens touching the row [gist.science section 2, gradient aggregation by
// averaging].  With token-importance weights lambda_t [sciencestack.ai
// contents: "Weighting MSE loss by token importance"] the loss of token t is
// lambda_t/2 ||out_t - y_t||^2: g_t is scaled by lambda_t, and a token with
// lambda_t = 0 emits no pairs (it reads only and is not counted).
//
// The k value rows are fetched as float4 per lane (coalesced 1 KiB per
// wave-load) and kept in registers for the backward when they fit.

#include "fwpkm.h"
#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

// Candidate c of the pruned Cartesian list for top-k, as (i << 8) | j: rows
// i = 0, 1, ... of floor(k / (i + 1)) candidates each, in order.  A table
// per k (it depends on k alone), so each lane's pair is one load issued with
// the kernel's first loads instead of a loop of divisions.
constexpr int kCartMax = 3 * kWave;     // sum_i floor(32 / i) = 130 candidates at most
struct CartTable {
  unsigned short ij[FWPKM_MAX_TOPK + 1][kCartMax];
};
constexpr CartTable make_cart_table() {
  CartTable t{};
  for (int k = 1; k <= FWPKM_MAX_TOPK; ++k) {
    int c = 0;
    for (int i = 0; i < k; ++i)
      for (int j = 0; j < k / (i + 1); ++j) t.ij[k][c++] = (unsigned short)((i << 8) | j);
  }
  return t;
}
__constant__ CartTable kCart = make_cart_table();

template <int KMAX, int VR, bool WRITE>
__global__ __launch_bounds__(kReadTokensMax * kWave) void kb_read(ChunkArgs a) {
  constexpr bool KEEP = KMAX * VR <= 32;
  // the launch arguments the first loads need, fetched in one batch with one
  // wait (left to itself the compiler fetches them in dependent rounds)
  asm volatile("" :: "s"(a.T), "s"(a.U), "s"(a.kb_tpw), "s"(a.kb_nbx), "s"(a.kb_div_nbx.m), "s"(a.kb_div_nbx.l),
               "s"(a.k), "s"(a.n),
               "s"(a.div_H.m), "s"(a.div_H.l), "s"(a.H), "s"(a.nblk), "s"(a.half_i), "s"(a.half_o),
               "s"(a.qnorm), "s"(a.tw), "s"(a.y), "s"(a.dv), "s"(a.mode));
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int nbx = a.kb_nbx;                           // workgroups per unit
  const int item = unit_affine_item(blockIdx.x, a.U, nbx);
  const int u = fast_div(item, a.kb_div_nbx);
  const int t = (item - u * nbx) * a.kb_tpw + wave;
  if (t >= a.T) return;
  const int k = a.k;
  const int n = a.n;
  const int b = fast_div(u, a.div_H), hh = u - b * a.H;
  const int64_t ut = (int64_t)u * a.T + t;
  const int64_t io = ((int64_t)(b * a.T + t) * a.H + hh);
  const int dv4 = a.dv >> 2;

  // loads that do not depend on the selection go out first, all together:
  // nothing here sits behind a branch (a load inside one is waited for on
  // its own), values a lane or mode does not use are masked afterwards.
  // Loads complete in issue order, so the candidate lists (wanted first, and
  // in this XCD's L2) go out before the target row (from HBM, wanted last).
  int ix[2];
  float ov[2];
  if (a.nblk == 1) {
    // lanes past k re-read entry 0 and are masked to the empty key
    const int li = lane < k ? lane : 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t base = (ut * 2 + h) * k;
      ix[h] = a.half_i[base + li];
      ov[h] = a.half_o[base + li];
    }
  }
  // this lane's Cartesian candidates (lane + 64 r); the table's rows are
  // zero past npr, and lanes past npr are masked below
  constexpr int J = 3;                        // sum_i floor(32/i) = 130 <= 3 * 64
  int cij[J];
#pragma unroll
  for (int r = 0; r < J; ++r) cij[r] = kCart.ij[k][lane + kWave * r];
  const float qn = (a.qnorm[ut * 2] + a.qnorm[ut * 2 + 1]) * (a.mode == 0 ? 1.f : 0.f);
  // token-importance weight of this token's loss; 0 = read only, no write.
  // Without weights the load reads this token's query norm instead (any
  // valid address), so that it never sits behind a branch.
  const bool has_tw = WRITE && a.tw != nullptr;
  const float lam_ld = *(has_tw ? a.tw + io : a.qnorm + ut * 2);
  const float lam = has_tw ? lam_ld : 1.0f;
  float4 yv[VR];
#pragma unroll
  for (int j = 0; j < VR; ++j) {
    yv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (WRITE) {
      // columns past the row re-read its last float4, zeroed when used
      const int c = lane + 64 * j;
      yv[j] = reinterpret_cast<const float4*>(a.y + io * a.dv)[c < dv4 ? c : dv4 - 1];
    }
  }

  // ---- 1. per-half best-k lists (lane m < k holds the m-th best), as
  // packed (ordering key, sub-key index) keys
  skey hk[2];
  if (a.nblk == 1) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned int m32 = opaque_mask(lane < k && ix[h] != kNoIndex);
      const skey m = (skey)m32 << 32 | m32;
      hk[h] = (pack_key(order_key(ov[h]), ix[h]) & m) | (kEmptyKey & ~m);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t base = (ut * 2 + h) * a.nblk * k;
    if (a.nblk != 1) {
      // merge the per-block lists, each sorted best-first: the best k so far
      // sit in lanes 0..k-1 (lanes k..KMAX-1 empty) and the next block's list
      // goes into lanes KMAX..2 KMAX-1 in reverse order, so that lanes
      // 0..2 KMAX-1 hold one bitonic sequence; a bitonic merge over 2 KMAX
      // lanes sorts it and the best k are back in lanes 0..k-1 (log2(2 KMAX)
      // exchange steps a block, where sorting a wave of candidates took 21).
      // The next block's loads are issued before this block's merge.
      static_assert(2 * KMAX <= kWave, "two lists fit the wave");
      const int nb = a.nblk;
      auto entry_of = [&](int blk) { return blk == 0 ? lane : 2 * KMAX - 1 - lane; };
      auto fetch = [&](int blk, int& ix, float& ov) {
        const int c = min(max(entry_of(blk), 0), k - 1);   // lanes without an entry re-read one, masked
        ix = a.half_i[base + (int64_t)blk * k + c];
        ov = a.half_o[base + (int64_t)blk * k + c];
      };
      int ixn;
      float ovn;
      fetch(0, ixn, ovn);
      skey x = kEmptyKey;
      for (int blk = 0; blk < nb; ++blk) {                  // block-uniform
        const int ix = ixn;
        const float ov = ovn;
        fetch(min(blk + 1, nb - 1), ixn, ovn);
        const int e = entry_of(blk);
        const bool slot_ok = blk == 0 ? lane < k : (lane >= KMAX && lane < 2 * KMAX && e < k);
        const unsigned int m32 = opaque_mask(slot_ok && ix != kNoIndex);
        const skey m = (skey)m32 << 32 | m32;
        const skey cand = (pack_key(order_key(ov), ix) & m) | (kEmptyKey & ~m);
        if (blk == 0) {
          x = cand;
        } else {
          x = lane < KMAX ? x : cand;
          key_merge_steps<2 * KMAX, 2 * KMAX, KMAX>(x);
          x = lane < k ? x : kEmptyKey;
        }
      }
      hk[h] = x;
    }
  }

  // ---- 2. pruned Cartesian candidates, then the k best
  const int npr = a.npr;
  skey sel;
  {
    const int jr = (npr + kWave - 1) / kWave;   // rounds that hold candidates (1 for k <= 20)
    skey cx[J];
#pragma unroll
    for (int r = 0; r < J; ++r) {
      cx[r] = kEmptyKey;
      if (r >= jr) continue;                     // wave-uniform
      const bool in = lane + 64 * r < npr;
      const int i = cij[r] >> 8, j = cij[r] & 255;
      const skey ka = __shfl(hk[0], i, kWave);
      const skey kb = __shfl(hk[1], j, kWave);
      const int ia = key_index(ka), ib = key_index(kb);
      // tie-break index (a << 12) | b orders exactly as the slot a*n + b does
      // (b < n <= 4096) and gives a and b back without a divide
      cx[r] = (in && ia != kNoIndex && ib != kNoIndex)
                  ? pack_key(order_key(key_value(ka) + key_value(kb)), (ia << 12) | ib)
                  : kEmptyKey;
    }
    if (npr <= 16) {
      sel = cx[0];
      sort_keys<16>(sel);
    } else if (npr <= 32) {
      sel = cx[0];
      sort_keys<32>(sel);
    } else if (npr <= 64) {
      sel = cx[0];
      sort_keys<64>(sel);
    } else {
      // k rounds of wave-wide minimum; lane r keeps the r-th best
      sel = kEmptyKey;
      for (int round = 0; round < k; ++round) {
        skey m = cx[0];
#pragma unroll
        for (int r = 1; r < J; ++r) m = cx[r] < m ? cx[r] : m;
        m = min_lanes(m);
#pragma unroll
        for (int r = 0; r < J; ++r) cx[r] = cx[r] == m ? kEmptyKey : cx[r];
        if (lane == round) sel = m;
      }
    }
  }
  const float sel_o = key_value(sel);
  const int sel_ab = key_index(sel);                          // (a << 12) | b
  const int sel_s = sel == kEmptyKey ? kNoIndex : (sel_ab >> 12) * n + (sel_ab & 4095);

  // ---- 3. weights (lanes m < k)
  const int64_t N = (int64_t)n * n;
  const bool active = lane < k && sel_s != kNoIndex;
  float w = 0.f, uinv = 0.f;
  if (a.mode == 0) {
    float D = qn + sel_o;
    D = D > 0.f ? D : 0.f;
    uinv = active ? 1.0f / (a.eps + D) : 0.f;
    const float s = wave_sum(uinv);
    w = uinv / s;
  } else {
    const float smax = -readlane_f(sel_o, 0);
    const float e = active ? expf(-sel_o - smax) : 0.f;
    const float s = wave_sum(e);
    w = e / s;
  }
  if (!active) w = 0.f;

  // ---- 4. gather-reduce of the k value rows
  const float* Vu = a.v + (int64_t)b * a.stride_v + (int64_t)hh * N * a.dv;
  float4 acc[VR];
#pragma unroll
  for (int j = 0; j < VR; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 rows[KEEP ? KMAX : 1][VR];
  if (KEEP) {
#pragma unroll
    for (int m = 0; m < KMAX; ++m) {
      if (m < k) {
        const int s = readlane_i(sel_s, m);
        const bool ok = s >= 0 && s < N;
        const float4* row = reinterpret_cast<const float4*>(Vu + (int64_t)(ok ? s : 0) * a.dv);
#pragma unroll
        for (int j = 0; j < VR; ++j) {
          const int c = lane + 64 * j;
          rows[KEEP ? m : 0][j] = (ok && c < dv4) ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < KMAX; ++m) {
      if (m < k) {
        const float wm = readlane_f(w, m);
#pragma unroll
        for (int j = 0; j < VR; ++j) {
          const float4 r = rows[KEEP ? m : 0][j];
          acc[j].x += wm * r.x; acc[j].y += wm * r.y; acc[j].z += wm * r.z; acc[j].w += wm * r.w;
        }
      }
    }
  } else {
    for (int m = 0; m < k; ++m) {
      const int s = readlane_i(sel_s, m);
      const bool ok = s >= 0 && s < N;
      const float wm = readlane_f(w, m);
      const float4* row = reinterpret_cast<const float4*>(Vu + (int64_t)(ok ? s : 0) * a.dv);
#pragma unroll
      for (int j = 0; j < VR; ++j) {
        const int c = lane + 64 * j;
        const float4 r = (ok && c < dv4) ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        acc[j].x += wm * r.x; acc[j].y += wm * r.y; acc[j].z += wm * r.z; acc[j].w += wm * r.w;
      }
    }
  }

  // ---- outputs of the read
  const int64_t ob = (int64_t)b * a.out_rows_b + (int64_t)t * a.H + hh;   // output row
  float4* ret = reinterpret_cast<float4*>(a.retrieved + ob * a.dv);
#pragma unroll
  for (int j = 0; j < VR; ++j) {
    const int c = lane + 64 * j;
    if (c < dv4) ret[c] = acc[j];
  }
  if (lane < k) {
    if (a.out_slots) a.out_slots[ob * k + lane] = sel_s;
    if (a.out_weights) a.out_weights[ob * k + lane] = w;
  }
#if FWPKM_DEVICE_CHECKS
  {
    bool twice = false;
    for (int m = 0; m < k; ++m) twice |= m < lane && readlane_i(sel_s, m) == sel_s;
    if (lane < k) {
      device_check(a, sel_s != kNoIndex, kChkCandidates);
      device_check(a, sel_s == kNoIndex || (sel_s >= 0 && sel_s < N), kChkSlot);
      device_check(a, !twice || sel_s == kNoIndex, kChkDistinct);
      device_check(a, w >= 0.f && w <= 1.f + 1e-6f, kChkWeight);   // false for NaN
    }
  }
#endif
  if (!WRITE) return;

  // ---- 5. backward
  float4* gw = reinterpret_cast<float4*>(a.g + ut * a.dv);
  float4 g[VR];
  float gout = 0.f;
#pragma unroll
  for (int j = 0; j < VR; ++j) {
    const int c = lane + 64 * j;
    g[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < dv4) {
      const float4 yy = yv[j];
      g[j] = make_float4(lam * (acc[j].x - yy.x), lam * (acc[j].y - yy.y),
                         lam * (acc[j].z - yy.z), lam * (acc[j].w - yy.w));
      gw[c] = g[j];
      gout += g[j].x * acc[j].x + g[j].y * acc[j].y + g[j].z * acc[j].z + g[j].w * acc[j].w;
    }
  }
  gout = wave_sum(gout);
  float gv_mine = 0.f;
  if (KEEP) {
#pragma unroll
    for (int m = 0; m < KMAX; ++m) {
      if (m < k) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < VR; ++j) {
          const float4 r = rows[KEEP ? m : 0][j];
          part += g[j].x * r.x + g[j].y * r.y + g[j].z * r.z + g[j].w * r.w;
        }
        part = wave_sum(part);
        if (lane == m) gv_mine = part;
      }
    }
  } else {
    for (int m = 0; m < k; ++m) {
      const int s = readlane_i(sel_s, m);
      const bool ok = s >= 0 && s < N;
      const float4* row = reinterpret_cast<const float4*>(Vu + (int64_t)(ok ? s : 0) * a.dv);
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < VR; ++j) {
        const int c = lane + 64 * j;
        const float4 r = (ok && c < dv4) ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        part += g[j].x * r.x + g[j].y * r.y + g[j].z * r.z + g[j].w * r.w;
      }
      part = wave_sum(part);
      if (lane == m) gv_mine = part;
    }
  }
  const float delta = w * (gv_mine - gout);
  const float c = (a.mode == 0) ? 2.0f * delta * uinv : delta;

  // ---- 6. pair lists: V (slot), K1 (row a), K2 (row b), merged per token
  const int am = active ? sel_ab >> 12 : n;
  const int bm = active ? sel_ab & 4095 : n;
  float sum1 = 0.f, sum2 = 0.f;
  bool first1 = true, first2 = true;
  for (int m = 0; m < k; ++m) {
    const int a2 = readlane_i(am, m);
    const int b2 = readlane_i(bm, m);
    const float c2 = readlane_f(c, m);
    if (a2 == am) { sum1 += c2; if (m < lane) first1 = false; }
    if (b2 == bm) { sum2 += c2; if (m < lane) first2 = false; }
  }
  if (lane < k) {
    const int64_t p = (int64_t)u * a.P + (int64_t)t * k + lane;
    const int64_t UP = (int64_t)a.U * a.P;
    const bool writes = active && lam != 0.f;   // a zero-weight token only reads
    a.keys[p] = writes ? sel_s : (int)N;   // N marks "no slot"; it sorts last
    a.sel_w[p] = w;
    const bool k1ok = writes && first1;
    const bool k2ok = writes && first2;
    a.keys[UP + p] = k1ok ? am : n;
    a.keys[2 * UP + p] = k2ok ? bm : n;
    a.coef[p] = k1ok ? sum1 : 0.f;
    a.coef[UP + p] = k2ok ? sum2 : 0.f;
  }
}

namespace {

template <int KMAX, int VR>
hipError_t launch_kb_t(const ChunkArgs& a, bool write, hipStream_t s, const LaunchTiming* tm) {
  const dim3 grid((unsigned)(a.kb_nbx * a.U));       // unit-major, see unit_affine_item
  const dim3 block((unsigned)(a.kb_tpw * kWave));
  if (write) return fw_launch(kb_read<KMAX, VR, true>, grid, block, 0, s, tm, a);
  return fw_launch(kb_read<KMAX, VR, false>, grid, block, 0, s, tm, a);
}

template <int KMAX>
hipError_t launch_kb_k(const ChunkArgs& a, bool write, hipStream_t s, const LaunchTiming* tm) {
  const int vr = ((a.dv >> 2) + 63) / 64;
  if (vr <= 1) return launch_kb_t<KMAX, 1>(a, write, s, tm);
  if (vr <= 2) return launch_kb_t<KMAX, 2>(a, write, s, tm);
  if (vr <= 4) return launch_kb_t<KMAX, 4>(a, write, s, tm);
  return launch_kb_t<KMAX, 8>(a, write, s, tm);
}

}  // namespace

hipError_t launch_kb(const ChunkArgs& args, bool write, hipStream_t s, const LaunchTiming* tm) {
  ChunkArgs a = with_divisors(args);
  // tokens per workgroup: the most (up to four) that still leaves a
  // workgroup for every compute unit.  Two-token workgroups spread the
  // library default's 512 tokens over all 256 units (read 9.7 -> 8.8 us);
  // from 2,048 tokens on, four-token ones reach every unit and the size
  // measured the same.
  a.kb_tpw = kReadTokensMax;
  while (a.kb_tpw > 1 && (int64_t)a.U * ((a.T + a.kb_tpw - 1) / a.kb_tpw) < 256) a.kb_tpw /= 2;
  a.kb_nbx = (a.T + a.kb_tpw - 1) / a.kb_tpw;
  a.kb_div_nbx = make_fastdiv(a.kb_nbx > 1 ? a.kb_nbx : 1);
  if (a.k <= 4) return launch_kb_k<4>(a, write, s, tm);
  if (a.k <= 8) return launch_kb_k<8>(a, write, s, tm);
  if (a.k <= 16) return launch_kb_k<16>(a, write, s, tm);
  return launch_kb_k<32>(a, write, s, tm);
}

}  // namespace fwpkm
