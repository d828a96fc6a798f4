// KF: the sequence-level layer around the chunk step.
//
// [PyPI page "fast-weight-product-key-memory", Usage: the memory module
// takes model-width tokens and carries its memories from call to call;
// gist.science "Fast-weight Product Key Memory", section 2, Core
// Architecture (Gated Residual Output) and Key Technical Choices (Lookahead
// Targets).]
//
//   kf_project  [q | v] = W_in x for every token: one fp32 GEMM on the
//               matrix cores (v_mfma_f32_16x16x4f32).  The epilogue writes
//               queries in the chunk-major layout the chunk step reads and
//               each token's value as the target of the token before it.
//   kf_prep     zero target and weight 0 for each sequence's last token
//               (no successor: it reads without writing), weight 1 for the
//               other tokens of the last chunk.
//   kf_gate     out = g r + (1 - g) x per head, g = sigmoid(w_gate[h] . x +
//               b_gate[h]), in place over the memory reads r.

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

namespace {

constexpr int kPM = 128;             // tokens per workgroup tile
constexpr int kPN = 128;             // output features per workgroup tile
constexpr int kPK = 32;              // input features staged per step
constexpr int kPPitch = kPK + 4;     // LDS row pitch (floats)
constexpr int kPThreads = 256;       // 4 waves, 2 x 2 of 64 x 64
constexpr int kPLoads = kPM * kPK / 4 / kPThreads;   // float4 per thread per operand
static_assert(kPM == kPN, "one loader mapping serves both operands");
static_assert(kPLoads * 4 * kPThreads == kPM * kPK, "whole float4 loads");
constexpr int kPStage = (kPM + kPN) * kPPitch;                       // floats per stage
constexpr size_t kPLdsBytes = sizeof(float) * 2 * kPStage;           // two stages
static_assert(2 * kPLdsBytes <= 160 * 1024, "two workgroups per compute unit");

// Native 4-vectors for the staged tiles (plain registers; copies of the
// HIP float4 struct through memory would keep them in scratch).
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// Masks a loaded value through an opaque word so that the load itself stays
// unconditional (a select on the value would let the compiler branch around
// the load, and every such branch waits for its load alone).
__device__ __forceinline__ f4 keep_if4(f4 v, bool ok) {
  unsigned int m = ok ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return __builtin_bit_cast(f4, __builtin_bit_cast(u4, v) & m);
}

}  // namespace

// One 128 x 128 tile of P = X W_in^T (tokens x features) per workgroup.
// Both operands are row-major with the contraction index contiguous, so the
// staged rows hold kPK consecutive input features of one token / one output
// feature.  Within a staged step the 32 features feed 8 MFMAs; lane group kq
// (lane / 16) supplies features kq*8 .. kq*8+7 (the same permutation on both
// operands, so the sum is unchanged), which lets each lane read its 8 values
// as two 16-byte LDS loads.
__global__ __launch_bounds__(kPThreads, 2) void kf_project(SeqArgs s) {
  // two stages of both operand tiles: step k reads stage k % 2 while the
  // tiles of step k + 1 are written to the other one
  extern __shared__ float kf_lds[];
  const int M = s.B * s.S, N = s.Nq + s.Nv, D = s.D;
  const int mtiles = (M + kPM - 1) / kPM, ntiles = (N + kPN - 1) / kPN;
  const int total = mtiles * ntiles;
  int tile = blockIdx.x;
  // consecutive workgroups land on different XCDs; give each XCD runs of
  // consecutive tiles so the N tiles of one token tile share its L2
  if (total % 8 == 0) tile = (tile % 8) * (total / 8) + tile / 8;
  const int mt = tile / ntiles, nt = tile - mt * ntiles;
  const int m0 = mt * kPM, n0 = nt * kPN;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int row = lane & 15, kq = lane >> 4;

  // loader: float4 f of the tile is row f / 8, column 4 (f % 8); rows past
  // the matrix are clamped (their products are never stored)
  const float* arow[kPLoads];
  const float* brow[kPLoads];
  int lds_off[kPLoads];
#pragma unroll
  for (int i = 0; i < kPLoads; ++i) {
    const int f = tid + i * kPThreads;
    const int r = f >> 3, c4 = f & 7;
    const int ma = min(m0 + r, M - 1), nb = min(n0 + r, N - 1);
    arow[i] = s.x + (int64_t)ma * D + c4 * 4;
    brow[i] = s.w_in + (int64_t)nb * D + c4 * 4;
    lds_off[i] = r * kPPitch + c4 * 4;
  }
  f4 pa[kPLoads], pb[kPLoads];
  auto fetch = [&](int k0) __attribute__((always_inline)) {
    // a float4 past D (D is a multiple of 4) reloads the row's last float4;
    // it is zeroed on A when staged
#pragma unroll
    for (int i = 0; i < kPLoads; ++i) {
      const int col = ((tid + i * kPThreads) & 7) * 4;
      const int off = (k0 + col < D) ? k0 : D - 4 - col;   // row + col + off stays in the row
      pa[i] = *reinterpret_cast<const f4*>(arow[i] + off);
      pb[i] = *reinterpret_cast<const f4*>(brow[i] + off);
    }
  };

  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto stage = [&](int k0, int buf) __attribute__((always_inline)) {
    float* As = kf_lds + buf * kPStage;
    float* Bs = As + kPM * kPPitch;
#pragma unroll
    for (int i = 0; i < kPLoads; ++i) {
      const int col = ((tid + i * kPThreads) & 7) * 4;
      *reinterpret_cast<f4*>(&As[lds_off[i]]) = keep_if4(pa[i], k0 + col < D);
      *reinterpret_cast<f4*>(&Bs[lds_off[i]]) = pb[i];
    }
  };
  fetch(0);
  stage(0, 0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < D; k0 += kPK, buf ^= 1) {
    const bool more = k0 + kPK < D;
    fetch(more ? k0 + kPK : k0);                 // the last step reloads (unused): no branch around loads
    // keep the next tile's loads ahead of this tile's matrix work
    __builtin_amdgcn_sched_barrier(0);
    const float* As = kf_lds + buf * kPStage;
    const float* Bs = As + kPM * kPPitch;
    float a[4][8], b[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* ar = &As[(wm * 64 + i * 16 + row) * kPPitch + kq * 8];
      const float* br = &Bs[(wn * 64 + i * 16 + row) * kPPitch + kq * 8];
      const f4 a0 = *reinterpret_cast<const f4*>(ar), a1 = *reinterpret_cast<const f4*>(ar + 4);
      const f4 b0 = *reinterpret_cast<const f4*>(br), b1 = *reinterpret_cast<const f4*>(br + 4);
      a[i][0] = a0.x; a[i][1] = a0.y; a[i][2] = a0.z; a[i][3] = a0.w;
      a[i][4] = a1.x; a[i][5] = a1.y; a[i][6] = a1.z; a[i][7] = a1.w;
      b[i][0] = b0.x; b[i][1] = b0.y; b[i][2] = b0.z; b[i][3] = b0.w;
      b[i][4] = b1.x; b[i][5] = b1.y; b[i][6] = b1.z; b[i][7] = b1.w;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][st], b[j][st], acc[i][j], 0, 0, 0);
    // the other stage was last read in the previous step, before the barrier
    // that ended it
    if (more) stage(k0 + kPK, buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds tokens m0 + wm*64 + i*16 + 4*kq + r, feature
  // n0 + wn*64 + j*16 + row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + 4 * kq + r;
      if (m >= M) continue;
      const int b = m / s.S, t = m - b * s.S;
      const int64_t qrow = seq_chunk_row(s, b, t);
      const int64_t yrow = t > 0 ? seq_chunk_row(s, b, t - 1) : -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + row;
        if (n < s.Nq) {
          s.q_all[qrow * s.Nq + n] = acc[i][j][r];
        } else if (n < N && yrow >= 0) {
          s.y_all[yrow * s.Nv + (n - s.Nq)] = acc[i][j][r];
        }
      }
    }
  }
}

// grid B: the last token of sequence b has no successor (zero target,
// weight 0); the other tokens of the last chunk have weight 1.
__global__ __launch_bounds__(256) void kf_prep(SeqArgs s) {
  const int b = blockIdx.x;
  const int64_t yrow = seq_chunk_row(s, b, s.S - 1);
  for (int j = threadIdx.x; j < s.Nv; j += blockDim.x) s.y_all[yrow * s.Nv + j] = 0.f;
  const int last0 = (s.S - 1) / s.C * s.C;
  const int cl = s.S - last0;
  for (int e = threadIdx.x; e < cl * s.H; e += blockDim.x)
    s.tw_last[(int64_t)b * cl * s.H + e] = (e / s.H == cl - 1) ? 0.f : 1.f;
}

// One wave per token: the gate of each head from the whole token, then that
// head's slice of the output.
__global__ __launch_bounds__(256) void kf_gate(SeqArgs s) {
  const int m = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
  const int lane = lane_id();
  if (m >= s.B * s.S) return;
  const int D4 = s.D / 4, dv4 = s.dv / 4;
  const float4* x4 = reinterpret_cast<const float4*>(s.x + (int64_t)m * s.D);
  float4* o4 = reinterpret_cast<float4*>(s.out + (int64_t)m * s.D);
  for (int h = 0; h < s.H; ++h) {
    const float4* w4 = reinterpret_cast<const float4*>(s.w_gate + (int64_t)h * s.D);
    float z = 0.f;
    for (int d = lane; d < D4; d += kWave) {
      const float4 xv = x4[d], wv = w4[d];
      z += xv.x * wv.x + xv.y * wv.y + xv.z * wv.z + xv.w * wv.w;
    }
    z = wave_sum(z) + (s.b_gate ? s.b_gate[h] : 0.f);
    const float g = 1.0f / (1.0f + expf(-z));
    for (int j = lane; j < dv4; j += kWave) {
      const float4 r = o4[h * dv4 + j], xv = x4[h * dv4 + j];
      o4[h * dv4 + j] = make_float4(g * r.x + (1.0f - g) * xv.x, g * r.y + (1.0f - g) * xv.y,
                                    g * r.z + (1.0f - g) * xv.z, g * r.w + (1.0f - g) * xv.w);
    }
  }
}

hipError_t launch_kf_project(const SeqArgs& s, hipStream_t st, const LaunchTiming* tm) {
  const int M = s.B * s.S, N = s.Nq + s.Nv;
  const int64_t tiles = (int64_t)((M + kPM - 1) / kPM) * ((N + kPN - 1) / kPN);
  // the last-token prep writes rows the projection never writes: either order works
  LaunchTiming first, last;
  if (tm) {
    first.beg = tm->beg;
    last.end = tm->end;
  }
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&kf_project),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPLdsBytes);
  if (attr != hipSuccess) return attr;
  hipError_t e = fw_launch(kf_project, dim3((unsigned)tiles), dim3(kPThreads), (uint32_t)kPLdsBytes, st,
                           tm ? &first : nullptr, s);
  if (e == hipSuccess) e = fw_launch(kf_prep, dim3(s.B), dim3(256), 0, st, tm ? &last : nullptr, s);
  return e;
}

hipError_t launch_kf_gate(const SeqArgs& s, hipStream_t st, const LaunchTiming* tm) {
  const int64_t M = (int64_t)s.B * s.S;
  return fw_launch(kf_gate, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, st, tm, s);
}

}  // namespace fwpkm
