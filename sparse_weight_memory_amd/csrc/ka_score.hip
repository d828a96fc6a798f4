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
// Each wave stages its own 16 key rows through a private LDS slice (a
// wave-wide load of matrix operands straight from memory would touch 16 key
// rows at once, which the load path serves at a fraction of its rate).
// When every chunk of the wave's dims is full, whole-line direct loads
// (global_load_lds_dwordx4) fill a ring of two 32-dim slots; otherwise
// chunks of 64 (or, for d_h > 256, 32) dims travel through registers into
// two LDS buffers.  With no barrier inside the contraction, the waves of a
// SIMD drift apart and one's LDS traffic overlaps another's matrix work.
// Key norms are summed in fp32 beside the contraction (on this chip fp32
// matrix instructions share the vector issue, so every extra instruction in
// that loop costs time): their rounding, ~1e-7 of ||K||^2, stays well below
// the dot product's and the 1e-6 relative gap at which candidates count as
// tied.
//
// Selection, one wave per token, on packed 64-bit (value, index) keys.  For
// blocks of 128 or 256 keys each lane first takes the smallest value of its
// candidates; the k-th smallest of those 64 values (a 32-bit bitonic sort)
// bounds the answer, only the candidates at or below it are compacted into
// LDS, and a 64-bit bitonic sort over 8, 16, 32 or 64 lanes orders them.  Where
// more than 64 pass (mass ties) and for 64-key blocks: a bitonic sort of the
// first 64 candidates gives a threshold (the k-th best), the remaining ones
// are filtered against it with one ballot per 64, and a bitonic sort of the
// k best plus the survivors gives the top-k.  Every step orders by (value,
// index), which is unique, so both give the same, deterministic result.
// Work items are laid out so that the token tiles sharing one key block run
// on one XCD (workgroup i is dispatched to XCD i % 8), which keeps the block's
// keys in that XCD's L2.

#include <algorithm>
#include <utility>

#include "fwpkm_device.h"
#include "fwpkm_launch.h"

namespace fwpkm {

typedef float v4f __attribute__((ext_vector_type(4)));

// Ascending bitonic sort of one 32-bit word per lane within every aligned
// group of GROUP lanes (32 or the whole wave).
template <int S>
__device__ __forceinline__ void cas_u32(unsigned int& x, bool ascending) {
  const unsigned int o = (unsigned int)xor_lane<S>((int)x);
  const bool keep_min = ((lane_id() & S) == 0) == ascending;
  x = keep_min ? min(x, o) : max(x, o);
}
template <int SIZE, int GROUP, int S>
__device__ __forceinline__ void u32_merge_steps(unsigned int& x) {
  cas_u32<S>(x, SIZE == GROUP || (lane_id() & SIZE) == 0);
  if constexpr (S > 1) u32_merge_steps<SIZE, GROUP, S / 2>(x);
}
template <int SIZE, int GROUP>
__device__ __forceinline__ void u32_stages(unsigned int& x) {
  if constexpr (SIZE > 2) u32_stages<SIZE / 2, GROUP>(x);
  u32_merge_steps<SIZE, GROUP, SIZE / 2>(x);
}
template <int GROUP = kWave>
__device__ __forceinline__ void sort_u32(unsigned int& x) { u32_stages<GROUP, GROUP>(x); }

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
__host__ __device__ inline int ka_chunks_of(int share) {
  const unsigned int nchunks = ((unsigned int)share + DC - 1) / DC;
  return (int)((nchunks + PF - 1) / PF * PF);
}

// dims of d_h per dim share of a wave
inline int ka_share(int half, int blk) {
  const int ndq = kScoreWaves / (blk / 16);
  return ((half + 16 * ndq - 1) / (16 * ndq)) * 16;
}

template <int DC, int PF>
inline int ka_chunks(int half, int blk) {
  return ka_chunks_of<DC, PF>(ka_share(half, blk));
}

// Width of a staged query row: every dim a chunk of any dim share may touch
// (columns past d_h are zero), so operand reads need no bounds test.
template <int DC, int PF>
__host__ __device__ inline int ka_query_width_of(int share, int ndq) {
  return (ndq - 1) * share + ka_chunks_of<DC, PF>(share) * DC;
}

template <int DC, int PF>
inline int ka_query_width(int half, int blk) {
  return ka_query_width_of<DC, PF>(ka_share(half, blk), kScoreWaves / (blk / 16));
}

// Key staging straight from global memory into LDS (kDma, only with kFull):
// each wave owns a ring of kPrefetch slots of 16 rows x kDimChunk dims.  One
// global_load_lds_dwordx4 fills 64 consecutive 16-byte LDS slots, so a slot's
// layout is row-major in load order; lane l of a load takes key row
// r = l / (kDimChunk / 4) (+ rows of earlier loads) and the dim group
// (l % (kDimChunk / 4)) ^ swz(r), which puts the 16 rows of a matrix-operand
// read in 16 different 16-byte bank groups.
template <int kDimChunk>
__device__ __forceinline__ int dma_swizzle(int r) {
  constexpr int kCols = kDimChunk / 4;          // float4 per staged row
  return (r / (16 / kCols)) % kCols;
}

// Byte offset of an LDS location (the pointer points into __shared__ memory).
__device__ __forceinline__ unsigned int lds_offset(const float* p) {
  return (unsigned int)(uintptr_t)(__attribute__((address_space(3))) const float*)p;
}

// 2 S 16-byte LDS reads (S key operands, S query operands) issued together,
// with the wait for all of them inside the same asm block, so no result is
// visible before it has arrived.  KOFF / QOFF are byte offsets added to every
// key / query address as the instructions' immediate offsets.
template <int S, int KOFF, int QOFF>
__device__ __forceinline__ void lds_read_wait(v4f (&ka)[S], v4f (&qa)[S], const unsigned int (&ka_at)[S],
                                              const unsigned int (&qa_at)[S]) {
#if __HIP_DEVICE_COMPILE__
  static_assert(S == 2 || S == 4, "two or four steps per chunk");
  static_assert(KOFF >= 0 && KOFF < 65536 && QOFF >= 0 && QOFF < 65536, "16-bit LDS offsets");
  if constexpr (S == 4) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\tds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\tds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%17\n\tds_read_b128 %5, %13 offset:%17\n\t"
        "ds_read_b128 %6, %14 offset:%17\n\tds_read_b128 %7, %15 offset:%17\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ka[0]), "=&v"(ka[1]), "=&v"(ka[2]), "=&v"(ka[3]),
          "=&v"(qa[0]), "=&v"(qa[1]), "=&v"(qa[2]), "=&v"(qa[3])
        : "v"(ka_at[0]), "v"(ka_at[1]), "v"(ka_at[2]), "v"(ka_at[3]),
          "v"(qa_at[0]), "v"(qa_at[1]), "v"(qa_at[2]), "v"(qa_at[3]), "i"(KOFF), "i"(QOFF));
  } else {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\tds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%9\n\tds_read_b128 %3, %7 offset:%9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ka[0]), "=&v"(ka[1]), "=&v"(qa[0]), "=&v"(qa[1])
        : "v"(ka_at[0]), "v"(ka_at[1]), "v"(qa_at[0]), "v"(qa_at[1]), "i"(KOFF), "i"(QOFF));
  }
#else
  (void)ka; (void)qa; (void)ka_at; (void)qa_at;
#endif
}

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 (an unrolled loop whose
// index is a compile-time constant).
template <class F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// s_waitcnt that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left alone).
template <int n>
__device__ __forceinline__ void wait_vm_at_most() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// kFull: every multiplied chunk lies inside its dim share and d_h (the
// shares tile d_h in whole chunks, and no ring padding is multiplied), so
// the staging loads need no mask.  kDma: stage keys with direct LDS loads
// (see dma_swizzle); kPrefetch is then the number of LDS slots per wave.
// Largest k whose selection takes two tokens per wave (32 lanes each).
constexpr int kPairMaxK = 16;

template <int kDimChunk, int kPrefetch, bool kFull, bool kDma>
__global__ __launch_bounds__(kScoreWaves * kWave) void ka_score_topk(ChunkArgs a) {
  static_assert(!kDma || kFull, "direct LDS staging cannot mask");
  constexpr int kKPitch = Staging<kDimChunk, kPrefetch>::kKPitch;
  constexpr int kStageF4 = Staging<kDimChunk, kPrefetch>::kStageF4;
  constexpr int kLanesPerRow = Staging<kDimChunk, kPrefetch>::kLanesPerRow;
  constexpr int kRowsPerLoad = Staging<kDimChunk, kPrefetch>::kRowsPerLoad;
  extern __shared__ float smem[];
  // every launch argument the prologue needs, as scalar operands of an empty
  // statement: they are fetched in one batch with one wait (left to itself
  // the compiler fetches them in three dependent rounds)
  asm volatile("" :: "s"(a.T), "s"(a.U), "s"(a.nblk), "s"(a.ka_ntt), "s"(a.H), "s"(a.half), "s"(a.key_block),
               "s"(a.ka_nkt_log2), "s"(a.ka_share), "s"(a.n), "s"(a.ka_div_ntt.m), "s"(a.ka_div_ntt.l),
               "s"(a.ka_div_nblk.m), "s"(a.ka_div_nblk.l), "s"(a.div_H.m), "s"(a.div_H.l), "s"(a.k1), "s"(a.k2),
               "s"(a.q), "s"(a.stride_k), "s"(a.dqk));
  const int half = a.half;
  // launch geometry from the host (shifts and multiply-shift divisions:
  // the prologue's scalar work is issued once per wave of the workgroup)
  const int blk = a.key_block;             // 64, 128 or 256
  const int blk_log2 = a.ka_nkt_log2 + 4;
  const int nkt = 1 << a.ka_nkt_log2;      // key tiles per block
  const int ndq = kScoreWaves >> a.ka_nkt_log2;   // dim shares per key tile
  const int share = a.ka_share;            // dims per share
  const int qwidth = ka_query_width_of<kDimChunk, kPrefetch>(share, ndq);
  const int qpitch = qwidth + 4;
  float* qs = smem;                                      // [16][qpitch]
  float* kst = qs + kTokTile * qpitch;                   // staged keys (register ring: [16 waves][2][16][kKPitch];
                                                         // direct: [16 waves][kPrefetch][16][kDimChunk])
  constexpr int kStageFloats = kDma ? kScoreWaves * kPrefetch * 16 * kDimChunk : 2 * kStageRows * kKPitch;
  double* knp = reinterpret_cast<double*>(kst + kStageFloats);  // [ndq][blk]
  // after the contraction the staging buffers are free:
  float* part = kst;                                     // [ndq][16][blk + 1]
  float* sc = part;                                      // [16][blk + 1], reuses part[0]
  constexpr int kSurvOffset = kDma ? 4 * kTokTile * (64 + 1) : kStageRows * kKPitch;
  static_assert(kSurvOffset * sizeof(float) + sizeof(skey) * kTokTile * kMaxBlk <= kStageFloats * sizeof(float),
                "survivors fit the staging area");
  skey* surv = reinterpret_cast<skey*>(kst + kSurvOffset);   // [16][blk] survivors

  const int ntt = a.ka_ntt;
  const int total = a.U * 2 * a.nblk * ntt;
  const int per_xcd = (int)(((unsigned int)total + 7) / 8);
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L >= total) return;
  const int r1 = fast_div(L, a.ka_div_ntt);
  const int tt = L - r1 * ntt;
  const int r2 = fast_div(r1, a.ka_div_nblk);
  const int kb = r1 - r2 * a.nblk;
  const int h = r2 & 1;
  const int u = r2 >> 1;
  const int b = fast_div(u, a.div_H), hh = u - b * a.H;
  const int t0 = tt * kTokTile;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();

  // ---- geometry: wave (kt, dq) = key tile kt over dim share dq
  const int kt = wave & (nkt - 1);
  const int dq = wave >> a.ka_nkt_log2;
  const int row = lane & 15;          // A row (key) / B column (token)
  const int quad = lane >> 4;         // 4-dim group inside a 16-dim step
  const int nchunks = (int)(((unsigned int)share + kDimChunk - 1) / kDimChunk);   // chunks holding data
  const int nchunks_p = ka_chunks_of<kDimChunk, kPrefetch>(share);            // chunks multiplied
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
  // direct staging: this wave's ring (a wave-uniform base, so the LDS
  // destination is set with scalar moves) and the per-lane byte offsets of a
  // chunk's loads; chunk c adds the scalar offset 4 c kDimChunk.  Buffer loads
  // over this unit's half table: an address past it reads zero.
  float* wring = kst + __builtin_amdgcn_readfirstlane(wave) * kPrefetch * 16 * kDimChunk;
  int dma_off[kStageF4];
#if __HIP_DEVICE_COMPILE__
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(kbase), (short)0, a.n * half * 4, 0x00020000);
#endif
  auto dma_issue = [&](int c, int slot) __attribute__((always_inline)) {
    // chunks past the end re-read chunk 0 into a slot nobody reads again
    const int cofs = c < nchunks ? c * kDimChunk * 4 : 0;
    float* dst = wring + slot * 16 * kDimChunk;
#if __HIP_DEVICE_COMPILE__   // a device builtin: the host pass only needs the kernel's stub
#pragma unroll
    for (int j = 0; j < kStageF4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krsrc, (__attribute__((address_space(3))) void*)(dst + j * kRowsPerLoad * kDimChunk), 16, dma_off[j],
          cofs, 0, 0);
#else
    (void)cofs;
    (void)dst;
#endif
  };
  const int half4 = half >> 2;
  const int qw4 = qwidth >> 2;
  // direct staging of the query tile too, when a row is whole 64-lane loads
  // (every staged column then lies inside d_h): wave w loads token t0 + w
  // into row w of the tile; rows past the chunk's last token lie past the
  // buffer's end and read zero
  const bool q_direct = kDma && qw4 % kWave == 0;
  if constexpr (kDma) {
#pragma unroll
    for (int j = 0; j < kStageF4; ++j) {
      const int r = j * kRowsPerLoad + lane / kLanesPerRow;
      const int gk = kb * blk + kt * 16 + r;
      const int col = (lane % kLanesPerRow) ^ dma_swizzle<kDimChunk>(r);
      dma_off[j] = ((gk < a.n ? gk : 0) * half + dq * share + col * 4) * 4;   // bytes
    }
    if (q_direct) {
      // issued ahead of the ring's chunks: loads retire in order, so the
      // tile is complete while the chunks are still in flight
#if __HIP_DEVICE_COMPILE__
      const int64_t qrow = (int64_t)a.H * a.dqk;               // floats between tokens
      const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.q + ((int64_t)(b * a.T + t0) * a.H + hh) * a.dqk + h * half), (short)0,
          (int)(((a.T - 1 - t0) * qrow + half) * 4), 0x00020000);
      float* qdst = qs + __builtin_amdgcn_readfirstlane(wave) * qpitch;
      const int qoff = (int)(__builtin_amdgcn_readfirstlane(wave) * qrow * 4);
      for (int m = 0; m < qw4 / kWave; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, (__attribute__((address_space(3))) void*)(qdst + m * 4 * kWave),
                                                 16, lane * 16 + m * 16 * kWave, qoff, 0, 0);
#endif
    }
#pragma unroll
    for (int i = 0; i + 1 < kPrefetch; ++i) dma_issue(i, i);    // in flight while queries are staged
  } else {
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) stage_load(stg[i], i);   // in flight while queries are staged
  }

  // ---- stage the 16-token query tile (this half) in LDS
  if (!q_direct) {
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
  }
  if constexpr (!kDma) {
    stage_store(stg[0], 0);
    stage_load(stg[0], kPrefetch);
    __syncthreads();
  } else {
    // this wave's query row has landed (only the ring's chunks may still be
    // in flight); __syncthreads() would also wait for those (vmcnt(0))
    if (q_direct) wait_vm_at_most<(kPrefetch - 1) * kStageF4>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // ---- query norms (fp64 sums), once per token and half; wave w <-> token w.
  // With direct staging they are stored after the contraction, so that only
  // key loads are outstanding while the loop counts them.
  auto query_norms = [&]() {
    if (kb == 0 && t0 + wave < a.T) {
      double s = 0.0;
      for (int d = lane; d < half; d += kWave) {
        const double x = qs[wave * qpitch + d];
        s += x * x;
      }
      s = wave_sum_d(s);
      if (lane == 0) a.qnorm[((int64_t)u * a.T + t0 + wave) * 2 + h] = (float)s;
    }
  };
  if constexpr (!kDma) query_norms();

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
  if constexpr (kDma) {
    // chunk c sits in slot c % kPrefetch; the loads of chunk c + kPrefetch - 1
    // refill the slot chunk c - 1 was read from (those reads fed the matrix
    // core already), then the wave waits until at most the newer chunks'
    // loads are outstanding: loads complete in order, so chunk c is in LDS.
    // The loop runs whole ring turns, so a chunk's slot is a constant and its
    // operand reads take fixed per-lane addresses plus immediate offsets.
    constexpr int kSteps = kDimChunk / 16;
    constexpr int kSlotBytes = 4 * 16 * kDimChunk;
    const int sw = dma_swizzle<kDimChunk>(row);
    unsigned int ka_at[kSteps], qa_at[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      ka_at[j] = lds_offset(&wring[row * kDimChunk + ((4 * j + quad) ^ sw) * 4]);
      qa_at[j] = lds_offset(&arow_base[j * 16 + quad * 4]);
    }
    for (int c0 = 0; c0 < nchunks_p; c0 += kPrefetch) {
      unsigned int qa_turn[kSteps];
#pragma unroll
      for (int j = 0; j < kSteps; ++j) qa_turn[j] = qa_at[j] + c0 * kSteps * 64;
      unroll_seq(
          [&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            dma_issue(c0 + s + kPrefetch - 1, (s + kPrefetch - 1) % kPrefetch);
            wait_vm_at_most<(kPrefetch - 1) * kStageF4>();
            // the chunk's operands in one block of LDS reads that waits for
            // them itself: read as ordinary loads, each would first wait for
            // every outstanding direct load (the compiler cannot tell the
            // slots apart)
            v4f akv[kSteps], bqv[kSteps];
            lds_read_wait<kSteps, s * kSlotBytes, s * kSteps * 64>(akv, bqv, ka_at, qa_turn);
#pragma unroll
            for (int j = 0; j < kSteps; ++j) {
              const v4f ak = akv[j];
              const v4f bq = bqv[j];
              ksq = fmaf(ak.x, ak.x, ksq); ksq = fmaf(ak.y, ak.y, ksq);
              ksq = fmaf(ak.z, ak.z, ksq); ksq = fmaf(ak.w, ak.w, ksq);
              acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.x, bq.x, acc0, 0, 0, 0);
              acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.z, bq.z, acc1, 0, 0, 0);
              acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.y, bq.y, acc0, 0, 0, 0);
              acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ak.w, bq.w, acc1, 0, 0, 0);
            }
          },
          std::make_integer_sequence<int, kPrefetch>{});
    }
    wait_vm_at_most<0>();   // the overrun loads land before the area is reused
    query_norms();
  } else {
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
        const int tok = e >> blk_log2, kk = e - (tok << blk_log2);
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
        const int tok = e >> blk_log2, kk = e - (tok << blk_log2);
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
      const int r = e >> blk_log2, c = e - (r << blk_log2);
      if (t0 + r < a.T && kb * blk + c < a.n) dst[(int64_t)r * a.addr_np + c] = sc[r * ppitch + c];
    }
  }

  // ---- the k best of the block, per token
  const int k = a.k;
  // one token on the whole wave: a filter on the lanes' best values and a
  // sort of the survivors, or the general path (mass ties, 64-key blocks)
  auto select_token = [&](int tl) __attribute__((always_inline)) {
    const int tw = t0 + tl;
    const float* srow = sc + tl * ppitch;
    auto cand = [&](int c) -> skey {
      const int gkey = kb * blk + c;
      return gkey < a.n ? pack_key(srow[c], gkey) : kEmptyKey;
    };
    skey x;
    bool picked = false;
    if (blk > kWave) {
      // Each lane's best candidate value bounds the answer: the k-th smallest
      // of those 64 values (compared on the value bits alone, a 32-bit sort)
      // is >= the k-th best key, so only candidates whose value bits do not
      // exceed it can be among the k best.  Those few get the exact 64-bit
      // sort.  When more than a wave's worth pass (mass ties, or fewer than k
      // real keys in the block) the general path below runs instead.
      constexpr int kR = kMaxBlk / kWave;
      const int nr = blk >> 6;
      skey cr[kR];
      unsigned int lo_hi = 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        cr[r] = r < nr ? cand(lane + r * kWave) : kEmptyKey;
        lo_hi = min(lo_hi, (unsigned int)(cr[r] >> 32));
      }
      sort_u32(lo_hi);
      const unsigned int th = (unsigned int)__builtin_amdgcn_readlane((int)lo_hi, k - 1);
      skey* sv = surv + tl * blk;
      int n = 0;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const bool pass = r < nr && (unsigned int)(cr[r] >> 32) <= th;
        const unsigned long long m = __ballot(pass);
        if (pass) sv[n + __popcll(m & ((1ull << lane) - 1ull))] = cr[r];
        n += __popcll(m);
      }
      if (n <= kWave) {
        x = lane < n ? sv[lane] : kEmptyKey;
        if (n <= 8) sort_keys<8>(x);
        else if (n <= 16) sort_keys<16>(x);
        else if (n <= 32) sort_keys<32>(x);
        else sort_keys<64>(x);
        picked = true;
      }
    }
    if (!picked) {
    x = cand(lane);
    sort_keys<64>(x);                               // the first 64, best first
    if (blk > kWave) {
      const skey th = readlane_k(x, k - 1);         // k-th best so far
      skey* sv = surv + tl * blk;
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
    }
    if (lane < k) {
      const int64_t base = ((((int64_t)u * a.T + tw) * 2 + h) * a.nblk + kb) * k;
      device_check(a, x == kEmptyKey || key_index(x) < a.n, kChkHalfIndex);
      a.half_o[base + lane] = key_value(x);
      a.half_i[base + lane] = key_index(x);
    }
  };

  if (blk > kWave && k <= kPairMaxK) {
    // Blocks of 128 or 256 keys: waves 0..7 take two tokens each, lanes
    // 32 g + l serving token 2 w + g, so half the waves sort half as many
    // lanes (the selection's cross-lane work shares each SIMD among fewer
    // waves).  Same bound as the one-token filter: the k-th smallest of the
    // 32 lanes' best value bits is >= the value bits of the k-th best key,
    // so every one of the k best passes; the survivors get the exact sort.
    if (wave >= kTokTile / 2 || t0 + 2 * wave >= a.T) return;   // wave-uniform
    const int g = lane >> 5, l = lane & 31;
    const int tl = 2 * wave + g;
    const float* srow = sc + tl * ppitch;
    constexpr int kR2 = kMaxBlk / 32;
    const int nr = blk >> 5;
    skey cr[kR2];
    unsigned int lo_hi = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < kR2; ++r) {
      const int c = l + 32 * r;
      const int gkey = kb * blk + c;
      cr[r] = (r < nr && gkey < a.n) ? pack_key(srow[c], gkey) : kEmptyKey;
      lo_hi = min(lo_hi, (unsigned int)(cr[r] >> 32));
    }
    sort_u32<32>(lo_hi);
    const unsigned int th0 = (unsigned int)__builtin_amdgcn_readlane((int)lo_hi, k - 1);
    const unsigned int th1 = (unsigned int)__builtin_amdgcn_readlane((int)lo_hi, 32 + k - 1);
    const unsigned int th = g ? th1 : th0;
    skey* sv = surv + tl * blk;
    const unsigned long long half_mask = g ? 0xFFFFFFFF00000000ull : 0xFFFFFFFFull;
    int n = 0;   // survivors of this lane's token
#pragma unroll
    for (int r = 0; r < kR2; ++r) {
      const bool pass = r < nr && (unsigned int)(cr[r] >> 32) <= th;
      const unsigned long long m = __ballot(pass) & half_mask;
      if (pass) sv[n + __popcll(m & ((1ull << lane) - 1ull))] = cr[r];
      n += __popcll(m);
    }
    const int n0 = __builtin_amdgcn_readlane(n, 0), n1 = __builtin_amdgcn_readlane(n, 32);
    const int nmax = max(n0, n1);
    skey x = l < n ? sv[l] : kEmptyKey;
    if (nmax <= 8) sort_keys<8>(x);
    else if (nmax <= 16) sort_keys<16>(x);
    else sort_keys<32>(x);
    // a token with more than 32 survivors takes the whole-wave path instead
    if (l < k && t0 + tl < a.T && n <= 32) {
      const int64_t base = ((((int64_t)u * a.T + t0 + tl) * 2 + h) * a.nblk + kb) * k;
      device_check(a, x == kEmptyKey || key_index(x) < a.n, kChkHalfIndex);
      a.half_o[base + l] = key_value(x);
      a.half_i[base + l] = key_index(x);
    }
    if (n0 > 32 && t0 + 2 * wave < a.T) select_token(2 * wave);
    if (n1 > 32 && t0 + 2 * wave + 1 < a.T) select_token(2 * wave + 1);
    return;
  }
  if (t0 + wave >= a.T) return;
  select_token(wave);
}

int score_key_block(int units, int tokens, int n) {
  const int ntt = (tokens + kTokTile - 1) / kTokTile;
  int blk = kMaxBlk;
  while (blk > 64 && (int64_t)units * 2 * ntt * ((n + blk - 1) / blk) < 256) blk /= 2;
  return blk;
}

template <int kDimChunk, int kPrefetch, bool kDma = false>
size_t ka_smem_bytes(int half, int blk) {
  constexpr int kKPitch = kDimChunk + 4;
  const int ndq = kScoreWaves / (blk / 16);
  // dim-share partials / scores and the filter survivors reuse the two key
  // staging buffers once the contraction is done
  static_assert(sizeof(float) * 4 * kTokTile * (64 + 1) <= sizeof(float) * kStageRows * kKPitch, "partials");
  static_assert(sizeof(skey) * kTokTile * kMaxBlk <= sizeof(float) * kStageRows * kKPitch, "survivors");
  const size_t staging = kDma ? sizeof(float) * kScoreWaves * kPrefetch * 16 * kDimChunk   // direct rings
                              : 2 * sizeof(float) * kStageRows * kKPitch;                 // double buffer
  return sizeof(float) * kTokTile * (ka_query_width<kDimChunk, kPrefetch>(half, blk) + 4)   // queries
         + staging                                                   // staged keys
         + sizeof(double) * ndq * blk;                               // key-norm partials
}

int ka_grid(const ChunkArgs& a) {
  const int ntt = (a.T + kTokTile - 1) / kTokTile;
  const int total = a.U * 2 * a.nblk * ntt;
  return 8 * ((total + 7) / 8);
}

namespace {

constexpr size_t kLdsBytes = 160 * 1024;

template <int DC, int PF, bool kFull, bool kDma = false>
hipError_t launch_ka_full(const ChunkArgs& a, hipStream_t s, const LaunchTiming* tm) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&ka_score_topk<DC, PF, kFull, kDma>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (attr != hipSuccess) return attr;
  return fw_launch(ka_score_topk<DC, PF, kFull, kDma>, dim3(ka_grid(a)), dim3(kScoreWaves * kWave),
                   (uint32_t)ka_smem_bytes<DC, PF, kDma>(a.half, a.key_block), s, tm, a);
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

hipError_t launch_ka(const ChunkArgs& args, hipStream_t s, const LaunchTiming* tm) {
  // the launch geometry the kernel takes ready-made
  ChunkArgs a = with_divisors(args);
  a.ka_ntt = (a.T + kTokTile - 1) / kTokTile;
  a.ka_nkt_log2 = 0;
  while ((16 << a.ka_nkt_log2) < a.key_block) ++a.ka_nkt_log2;   // key_block = 16 << log2, a power of two
  a.ka_share = ka_share(a.half, a.key_block);
  a.ka_div_ntt = make_fastdiv(std::max(1, a.ka_ntt));
  a.ka_div_nblk = make_fastdiv(std::max(1, a.nblk));
  {
    // full shapes (every 32-dim chunk of a share inside d_h, whole ring
    // turns of two slots) stage keys straight into LDS when the rings fit.
    // Two slots rather than four: at d_h <= 128 two workgroups then fit a
    // compute unit, so that one's selection and prologue overlap the other's
    // contraction when the grid runs in several rounds, and with one
    // workgroup per unit the deeper ring gains nothing measurable.
    const int ndq = kScoreWaves / (a.key_block / 16);
    const int share = ((a.half + 16 * ndq - 1) / (16 * ndq)) * 16;
    const bool full32 = share % 32 == 0 && ndq * share <= a.half;
    if (full32 && (share / 32) % 2 == 0 && ka_smem_bytes<32, 2, true>(a.half, a.key_block) <= kLdsBytes)
      return launch_ka_full<32, 2, true, true>(a, s, tm);
  }
  // wider chunks halve the barriers per contraction; they fit for d_h <= 256.
  // A ring deeper than the chunk count would only multiply zeros.
  if (ka_smem_bytes<64, 2>(a.half, a.key_block) <= kLdsBytes) {
    if (ka_chunks<64, 1>(a.half, a.key_block) == 1) return launch_ka_as<64, 1>(a, s, tm);
    return launch_ka_as<64, 2>(a, s, tm);
  }
  return launch_ka_as<32, 4>(a, s, tm);
}

}  // namespace fwpkm
