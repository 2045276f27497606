// Pooled block scores (FlashPrefill summary "长上下文加速 28 倍", 3.1: query
// blocks are scored against mean-pooled keys; inside each (query block, key
// block) tile the logits are normalised by their maximum, exponentiated and
// summed; the row is later re-aligned to its top key block).
//
// For KV head h and query block I the rows are every (query head of the
// group, token of I): R = g * n_I rows.  Output per J <= I:
//     L_IJ = M_IJ + ln S_IJ,  M_IJ = max_r x_rJ,  S_IJ = sum_r exp(x_rJ - M_IJ)
// with x_rJ = softmax_scale * q_r . kbar_J.
//
// gfx950 design:
//   * one workgroup (8 waves) owns one (h, I) and ALL its rows (small
//     launches split the key tiles of a row over several workgroups, since
//     columns are independent); the rows go
//     in passes of 8 waves x 2 chunks x 32 rows, each wave holding the Q
//     fragments of its two chunks in registers for the whole pass, so Q is
//     read from HBM once (passes = g / 4).
//   * pooled keys s_J = bf16(softmax_scale log2(e) kbar_J) (scaled in float64
//     and rounded once by the pooling pass, L2-resident) stream through
//     double-buffered LDS in tiles of 128 keys, copied with
//     global_load_lds_dwordx4 (no staging registers) into XOR-swizzled 256-B
//     rows, so the MFMA operand reads are conflict-free.
//   * X = Q . S^T on v_mfma_f32_32x32x16_bf16 with fp32 accumulation: the
//     log2-domain logits come straight out of the matrix core (e4m3 queries:
//     times the head's q_scale).  In the result layout a lane owns one
//     pooled-key column and 16 rows of each chunk: the exp-sum is lane-local,
//     lanes l and l^32 are merged with one v_permlane32_swap, and the 8 waves
//     through LDS once per tile.
//   * no column max: max_r |q_r|_2 * |s_J|_2 bounds every logit of column J
//     (Cauchy-Schwarz).  When that bound is at most kDirectMax for every
//     column of the row (bf16 / fp32 queries), the exp2-sums run on the
//     logits as they are, one exp and one add per element (no term can
//     overflow); otherwise against the bound as a per-column reference,
//     S = sum_r 2^(x_rJ - ref), L = ref + log2 S.  A wave whose sum for a
//     column falls below 2^-64 recomputes that chunk against its true max,
//     so the result keeps the same fp32 accuracy.
//   * error bound instead of a second MFMA term: rounding s_J to bf16 moves
//     x_rJ by at most |q_r|_2 * |lscale kbar_J - s_J|_2 (Cauchy-Schwarz), and
//     a log-sum-exp over rows moves by at most the largest such shift.  The
//     kernel writes that bound per score row (largest query-row norm of the
//     row times the largest residual bound of its key blocks, from the
//     pooling pass); the selection re-evaluates in float64 every entry the
//     bound cannot decide.
//   * software pipeline inside a wave: the MFMAs of key chunk j+1 (second
//     accumulator set) are independent of the exp-sums of chunk j, so the
//     matrix core and the VALU overlap; masking runs only for the ragged last
//     block.
#include <algorithm>

#include "fp_internal.hpp"

namespace fp {

namespace {

constexpr int kWaves = 8;
constexpr int kRC = 2;                         // 32-row chunks per wave per pass
constexpr int kChunksPerPass = kWaves * kRC;   // 512 rows per pass
constexpr int kJT = 128;                       // pooled keys per LDS tile
constexpr int kJC = kJT / 32;                  // 32-key chunks per tile
constexpr int kTerm = kJT * kHeadDim;          // bf16 elements of one term of a tile
constexpr float kLn2 = 0.6931471805599453f;

struct ScoresSmem {
  u16 kb[2][kTerm];              // [buffer]: 64 KiB
  float bn[2][kJT];              // [buffer]: |s_J|_2 of the tile's keys
  float2 part[2][kWaves][kJT];   // per wave (reference, sum) of each key, by buffer
  float red[3][kWaves];          // per wave: largest residual bound, largest row norm^2,
                                 // largest |s_J|_2
};
constexpr size_t kScoresSmem = sizeof(ScoresSmem);

struct ScoresArgs {
  SeqMap m;
  const void* q;
  const float* q_scale;
  const u16* kmean16;   // s_J = bf16(softmax_scale log2(e) kbar_J) [Hkv, NK, 128]
  const float* kres;    // residual bound of each pooled key [Hkv, NK] (log2 units)
  const float* bnorm;   // |s_J|_2 of each pooled key [Hkv, NK] (rounded up)
  float* scores;
  float* errb;          // per score row: bound on the error of its entries
  int64_t num_blocks;   // NK (pooled rows per KV head)
  int64_t num_qblocks;  // NQ (score rows per KV head)
  int hq, hkv, group, max_blocks;  // group: query heads per index list (1 per query head)
  int lists, kvdiv;                // list owners (score rows per query block); owner o
                                   // reads the pooled keys of KV head o / kvdiv
  int cparts;           // workgroups per (kv head, query block), each over a range of key tiles
};

// Q fragment of one 32-row chunk: lane l holds row l%32, head-dim elements
// [64*(l/32) + 8*kk, +8) for kk = 0..7 (the MFMA K index is a permutation of
// the head dim, applied identically to both operands).
template <int QDT>
__device__ __forceinline__ void load_q_frag(const void* q, int64_t row_elem, bool valid, int half,
                                            bf16x8* f) {
  if (!valid) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) f[kk] = bf16x8{};
    return;
  }
  const int64_t e0 = row_elem + 64 * half;
  if constexpr (QDT == FP_BF16) {
    const bf16x8* p = reinterpret_cast<const bf16x8*>(reinterpret_cast<const u16*>(q) + e0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) f[kk] = p[kk];
  } else if constexpr (QDT == FP_E4M3) {
    const uint2* p = reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(q) + e0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint2 w = p[kk];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        f[kk][i] = f32_to_bf16(e4m3_to_f32(((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu));
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + e0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const float4 a = p[2 * kk], b = p[2 * kk + 1];
      f[kk] = bf16x8{f32_to_bf16(a.x), f32_to_bf16(a.y), f32_to_bf16(a.z), f32_to_bf16(a.w),
                     f32_to_bf16(b.x), f32_to_bf16(b.y), f32_to_bf16(b.z), f32_to_bf16(b.w)};
    }
  }
}

// X chunk of 32 pooled keys (rows jc*32 .. +31 of the LDS tile) against the
// wave's kRC row chunks: 8 head-dim steps.  Chunks without valid
// rows hold zero Q fragments and are computed anyway (their results are
// masked), which keeps the instruction stream branch-free.
__device__ __forceinline__ void mma_chunk(const u16* bh, int jc, int col, int half,
                                          const bf16x8 (&qf)[kRC][8], f32x16* acc) {
  const int r = jc * 32 + col;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int off = r * kHeadDim + swz16(8 * half + kk, r) * 8;
    const bf16x8 vh = *reinterpret_cast<const bf16x8*>(bh + off);
#pragma unroll
    for (int rc = 0; rc < kRC; ++rc)
      acc[rc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rc][kk], vh, kk ? acc[rc] : f32x16{}, 0, 0, 0);
  }
}

// Column max / exp-sum of one 32-key chunk over this wave's rows, merged over
// the lane pair.  MASKED handles chunks with rows past the end of the block or
// past the last head (rows of this lane: m = 8*(i/4) + 4*half + (i%4)); a
// wave without any valid row yields (-inf, 0).
template <bool MASKED>
__device__ __forceinline__ float2 column_stats(const f32x16* acc, const float* csc,
                                               const int* nval, int half) {
  float m = -INFINITY;
#pragma unroll
  for (int rc = 0; rc < kRC; ++rc) {
    float mr = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      mr = fmaxf(mr, (!MASKED || row < nval[rc]) ? acc[rc][i] : -INFINITY);
    }
    m = fmaxf(m, mr * csc[rc]);  // scales are positive; -inf stays -inf
  }
  m = pair_max(m);
  float s = 0.f;
#pragma unroll
  for (int rc = 0; rc < kRC; ++rc) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      const float e = __builtin_amdgcn_exp2f(fmaf(acc[rc][i], csc[rc], -m));
      s += (!MASKED || row < nval[rc]) ? e : 0.f;
    }
  }
  return make_float2(m, pair_sum(s));
}

// Slice KK (0..7) of the column exp-sum of one finished 32-key chunk, spread
// over the eight head-dim steps of the next chunk's MFMAs: four of the 32
// (row chunk, row) elements per slice, in order.  DIRECT: sum of 2^x (every
// logit of the pass at most kDirectMax, csc = 1); otherwise sum of
// 2^(x csc - ref) against the column's reference ref (an upper bound of every
// logit of the column).
template <bool MASKED, bool DIRECT, int KK>
__device__ __forceinline__ void sum_slice(const f32x16* acc, const float* csc, const int* nval,
                                          int half, float ref, float& s) {
  if constexpr (KK == 0) s = 0.f;
#pragma unroll
  for (int e = 4 * KK; e < 4 * KK + 4; ++e) {
    const int rc = e >> 4, i = e & 15;
    const int row = 8 * (i >> 2) + 4 * half + (i & 3);
    const float x = __builtin_amdgcn_exp2f(DIRECT ? acc[rc][i] : fmaf(acc[rc][i], csc[rc], -ref));
    s += (!MASKED || row < nval[rc]) ? x : 0.f;
  }
}

// Largest logit bound (log2 units) for which the exp-sums run without a
// reference: a term is then at most 2^112 and a column of a pass sums at most
// 512 of them, so no sum overflows.
constexpr float kDirectMax = 112.f;

// A column's exp-sum against its reference is trusted when it is at least
// kSumFloor: its largest term is then >= 2^-75, a normal float, and terms
// flushed below 2^-126 change it by less than 2^-51 relatively.  Otherwise
// (a reference far above every logit of the column, or no valid row) the
// wave recomputes the chunk's statistics with the true column max.
constexpr float kSumFloor = 0x1p-64f;

// MFMAs of head-dim step kk of one 32-key chunk.
__device__ __forceinline__ void mma_step(const bf16x8 (&qf)[kRC][8], int kk, bf16x8 vh,
                                         f32x16* acc) {
#pragma unroll
  for (int rc = 0; rc < kRC; ++rc)
    acc[rc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rc][kk], vh, kk ? acc[rc] : f32x16{}, 0, 0, 0);
}

// One 32-key chunk's MFMAs with the statistics of the previous chunk woven
// in: per head-dim step, the operand of the next step is read from LDS, the
// two MFMAs issue one by one, each followed by a share of the statistics
// (independent VALU work that the in-order wave issues while the matrix core
// runs).  Scheduling fences between steps keep this order.
template <bool MASKED, bool DIRECT>
__device__ __forceinline__ float2 chunk_overlapped(const u16* bh, int jc, int col,
                                                   int half, const bf16x8 (&qf)[kRC][8],
                                                   f32x16* acc, const f32x16* prev,
                                                   const float* csc, const int* nval, float ref) {
  const int r = jc * 32 + col;
  auto opnd = [&](const u16* b, int kk) {
    return *reinterpret_cast<const bf16x8*>(b + r * kHeadDim + swz16(8 * half + kk, r) * 8);
  };
  float s;
  bf16x8 vh = opnd(bh, 0);
#define FP_STEP(KK)                                          \
  {                                                          \
    bf16x8 nh;                                               \
    if constexpr (KK < 7) nh = opnd(bh, KK + 1);             \
    mma_step(qf, KK, vh, acc);                               \
    sum_slice<MASKED, DIRECT, KK>(prev, csc, nval, half, ref, s); \
    interleave<2, 1>();                                      \
    __builtin_amdgcn_sched_barrier(0);                       \
    if constexpr (KK < 7) vh = nh;                           \
  }
  FP_STEP(0) FP_STEP(1) FP_STEP(2) FP_STEP(3) FP_STEP(4) FP_STEP(5) FP_STEP(6) FP_STEP(7)
#undef FP_STEP
  return make_float2(DIRECT ? 0.f : ref, pair_sum(s));
}

// Statistics of a finished chunk against the column reference, falling back
// to the true column max (column_stats) when any lane's sum is below
// kSumFloor (wave-uniform branch; acc must still hold the chunk).
template <bool MASKED>
__device__ __forceinline__ float2 checked(float2 st, const f32x16* acc, const float* csc,
                                          const int* nval, int half) {
  if (__builtin_expect(__any(!(st.y >= kSumFloor)), 0)) {
    bool rows = !MASKED;  // wave-uniform: a wave without any valid row yields (-inf, 0)
#pragma unroll
    for (int rc = 0; rc < kRC; ++rc) rows |= nval[rc] > 0;
    st = rows ? column_stats<MASKED>(acc, csc, nval, half) : make_float2(-INFINITY, 0.f);
  }
  return st;
}

// The same sums without interleaving (chunks outside the pipeline), with the
// same fallback.
template <bool MASKED, bool DIRECT>
__device__ __forceinline__ float2 ref_stats(const f32x16* acc, const float* csc, const int* nval,
                                            int half, float ref) {
  float s;
  sum_slice<MASKED, DIRECT, 0>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 1>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 2>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 3>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 4>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 5>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 6>(acc, csc, nval, half, ref, s);
  sum_slice<MASKED, DIRECT, 7>(acc, csc, nval, half, ref, s);
  return checked<MASKED>(make_float2(DIRECT ? 0.f : ref, pair_sum(s)), acc, csc, nval, half);
}

// One LDS tile for this wave.  Full tiles (kJC chunks) run as one basic block
// with two accumulator sets: chunk j+1's MFMAs overlap chunk j's statistics.
// ref[jc]: the reference of this lane's key column in chunk jc (unused when
// DIRECT).
template <bool MASKED, bool DIRECT>
__device__ __forceinline__ void tile_chunks(const u16* bh, int njc, int col,
                                            int half, const bf16x8 (&qf)[kRC][8],
                                            const float* csc, const int* nval, const float* ref,
                                            float2* part) {
  f32x16 acc0[kRC], acc1[kRC];
  if (njc == kJC) {
    static_assert(kJC == 4, "pipeline below is written for 4 chunks per tile");
    mma_chunk(bh, 0, col, half, qf, acc0);
    __builtin_amdgcn_sched_barrier(0);
    // each chunk's sums are checked before its accumulators are reused
    const float2 s0 = checked<MASKED>(
        chunk_overlapped<MASKED, DIRECT>(bh, 1, col, half, qf, acc1, acc0, csc, nval, ref[0]),
        acc0, csc, nval, half);
    const float2 s1 = checked<MASKED>(
        chunk_overlapped<MASKED, DIRECT>(bh, 2, col, half, qf, acc0, acc1, csc, nval, ref[1]),
        acc1, csc, nval, half);
    const float2 s2 = checked<MASKED>(
        chunk_overlapped<MASKED, DIRECT>(bh, 3, col, half, qf, acc1, acc0, csc, nval, ref[2]),
        acc0, csc, nval, half);
    const float2 s3 = ref_stats<MASKED, DIRECT>(acc1, csc, nval, half, ref[3]);
    if (half == 0) {
      part[col] = s0;
      part[32 + col] = s1;
      part[64 + col] = s2;
      part[96 + col] = s3;
    }
  } else {
    for (int jc = 0; jc < njc; ++jc) {
      mma_chunk(bh, jc, col, half, qf, acc0);
      const float2 st = column_stats<MASKED>(acc0, csc, nval, half);
      if (half == 0) part[jc * 32 + col] = st;
    }
  }
}

template <int QDT>
__global__ __launch_bounds__(512) void scores_kernel(ScoresArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  ScoresSmem& sm = *reinterpret_cast<ScoresSmem*>(smem_raw);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // heaviest rows (largest I of a sequence) first; the cparts workgroups of
  // a row take contiguous ranges of its key tiles (columns are independent)
  const int part = (int)(blockIdx.x % a.cparts);
  const int64_t item = (int64_t)a.lists * a.num_qblocks - 1 - blockIdx.x / a.cparts;
  const int h = (int)(item % a.lists);  // list owner
  const int gq = (int)(item / a.lists);
  const QBlock qb = query_block(a.m, gq);
  const int I = qb.I;
  const int nI = qb.nI;
  const int64_t tok0 = qb.tok0;
  const u16* kbase = a.kmean16 + ((int64_t)(h / a.kvdiv) * a.num_blocks + qb.kb0) * kHeadDim;
  float* out_row = a.scores + ((int64_t)h * a.num_qblocks + gq) * a.max_blocks;
  const int ncols = I + 1;
  const int ntiles_row = (ncols + kJT - 1) / kJT;
  const int tile0 = (int)(((int64_t)part * ntiles_row) / a.cparts);
  const int tile1 = (int)(((int64_t)(part + 1) * ntiles_row) / a.cparts);
  if (tile0 >= tile1) return;  // whole workgroup: no barrier is skipped by part of it
  const int nchunks = 4 * a.group;  // 32-row chunks: (head, 32-token slice)

  // Tile t = 32 segments of 1 KiB (4 key rows each); wave w issues segments
  // 4w .. 4w+3.  Lane i of a segment copies physical chunk i%16 of key row
  // 4*seg + i/16, i.e. logical chunk swz16(i%16, row).  Key rows past the
  // causal range re-read the last valid row (results unused).  The lane index
  // is made opaque here so that the source addresses are recomputed per tile
  // instead of being hoisted into live registers.
  const float* bnbase = a.bnorm + (int64_t)(h / a.kvdiv) * a.num_blocks + qb.kb0;
  auto stage = [&](int tile, int buf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int seg = wave * 4 + it;
      const int r = 4 * seg + (ln >> 4);
      const int J = min(tile * kJT + r, ncols - 1);
      const u16* src = kbase + (int64_t)J * kHeadDim + swz16(ln & 15, r) * 8;
      load_lds16(src, &sm.kb[buf][seg * 512]);
    }
    if (wave < 2) {  // the norms of the tile's 128 keys: one dword per lane
      const int J = min(tile * kJT + 64 * wave + ln, ncols - 1);
      __builtin_amdgcn_global_load_lds((gbl_void*)(bnbase + J), (lds_void*)&sm.bn[buf][64 * wave], 4, 0, 0);
    }
  };

  float qn2 = 0.f;  // largest squared query-row norm (q_scale included), all passes


  for (int pass = 0; pass * kChunksPerPass < nchunks; ++pass) {
    // ---- Q fragments of this pass (read once) ----
    bf16x8 qf[kRC][8];
    float csc[kRC], qsf[kRC];
    int nval[kRC];
    bool masked = false;
#pragma unroll
    for (int rc = 0; rc < kRC; ++rc) {
      const int c = pass * kChunksPerPass + rc * kWaves + wave;
      const int hh = c >> 2;
      const int t0 = 32 * (c & 3);
      const bool head_ok = c < nchunks;
      nval[rc] = head_ok ? max(0, min(32, nI - t0)) : 0;
      masked |= nval[rc] < 32;
      const int hq_idx = h * a.group + (head_ok ? hh : 0);
      const bool rvalid = col < nval[rc];
      const int64_t row_elem = ((tok0 + t0 + col) * a.hq + hq_idx) * (int64_t)kHeadDim;
      load_q_frag<QDT>(a.q, row_elem, rvalid, half, qf[rc]);
      qsf[rc] = QDT == FP_E4M3 ? a.q_scale[hq_idx] : 1.f;
      csc[rc] = qsf[rc];  // the keys carry softmax_scale log2(e)
    }
    // the first key tile does not depend on Q: in flight together with it
    stage(tile0, tile0 & 1);
    if (pass == 0) {
      // largest residual bound and largest |s_J| of the row's key blocks
      // (published by the barrier below), loads in flight with the Q loads
      const float* kres = a.kres + (int64_t)(h / a.kvdiv) * a.num_blocks + qb.kb0;
      float dm = 0.f, bm = 0.f;
      for (int J = (int)threadIdx.x; J < ncols; J += 64 * kWaves) {
        dm = fmaxf(dm, kres[J]);
        if constexpr (QDT != FP_E4M3) bm = fmaxf(bm, bnbase[J]);  // e4m3: never direct
      }
      dm = wave_max(dm);
      bm = wave_max(bm);
      if (lane == 0) {
        sm.red[0][wave] = dm;
        sm.red[2][wave] = bm;
      }
    }
    {
      // squared norms of this wave's rows (lanes l and l^32 hold the halves)
      float wn = 0.f;
#pragma unroll
      for (int rc = 0; rc < kRC; ++rc) {
        float n2 = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = (float)qf[rc][kk][i];
            n2 = fmaf(v, v, n2);
          }
        n2 = pair_sum(n2) * (qsf[rc] * qsf[rc]);
        wn = fmaxf(wn, n2);
      }
      wn = wave_max(wn);
      if (lane == 0) sm.red[1][wave] = wn;
    }

    wait_vm();
    __syncthreads();
    float qp2 = 0.f, bmax = 0.f;  // largest squared query-row norm of this pass, largest |s_J|
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      qp2 = fmaxf(qp2, sm.red[1][w]);
      bmax = fmaxf(bmax, sm.red[2][w]);
    }
    qn2 = fmaxf(qn2, qp2);
    // reference of a key column: max_r |q_r| |s_J| bounds every logit x_rJ of
    // the pass (Cauchy-Schwarz; the margin covers the fp32 accumulation and
    // roundings), so exp2(x_rJ - ref) <= ~1.  Below kDirectMax for every
    // column of the row, the sums need no reference (bf16 / fp32 queries,
    // whose logits carry no per-head scale).
    const float cref = __fsqrt_rn(qp2) * (1.f + 0x1p-10f);
    const bool direct = QDT != FP_E4M3 && cref * bmax <= kDirectMax;

    for (int tile = tile0; tile < tile1; ++tile) {
      const int buf = tile & 1;
      if (tile + 1 < tile1) stage(tile + 1, buf ^ 1);
      const int njc = min(kJC, (ncols - tile * kJT + 31) >> 5);
      const u16* bh = sm.kb[buf];
      float ref[kJC];
      if (direct) {
#pragma unroll
        for (int jc = 0; jc < kJC; ++jc) ref[jc] = 0.f;
        if (masked)
          tile_chunks<true, true>(bh, njc, col, half, qf, csc, nval, ref, sm.part[buf][wave]);
        else
          tile_chunks<false, true>(bh, njc, col, half, qf, csc, nval, ref, sm.part[buf][wave]);
      } else {
#pragma unroll
        for (int jc = 0; jc < kJC; ++jc) ref[jc] = cref * sm.bn[buf][jc * 32 + col];
        if (masked)
          tile_chunks<true, false>(bh, njc, col, half, qf, csc, nval, ref, sm.part[buf][wave]);
        else
          tile_chunks<false, false>(bh, njc, col, half, qf, csc, nval, ref, sm.part[buf][wave]);
      }

      wait_vm();
      __syncthreads();

      if (threadIdx.x < kJT) {
        const int J = tile * kJT + (int)threadIdx.x;
        if (J < ncols) {
          float m = -INFINITY;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sm.part[buf][w][threadIdx.x].x);
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            const float2 p = sm.part[buf][w][threadIdx.x];
            sum += p.y * __builtin_amdgcn_exp2f(p.x - m);  // inactive waves: (-inf, 0)
          }
          // log2 domain -> natural log; passes after the first merge with the
          // value already stored
          float L = (m + __log2f(sum)) * kLn2;
          if (pass > 0) {
            const float P = out_row[J];
            const float hi = fmaxf(P, L);
            L = hi + __logf(__expf(P - hi) + __expf(L - hi));
          }
          out_row[J] = L;
        }
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    // every entry of the row: |L_fast - L| <= ln 2 * max_r |q_r| * max_J
    // kres_J (+ the fp32 rounding of the statistics; kres is in log2 units,
    // L in natural log); the factor covers the rounding of the bound itself.
    // Workgroups sharing a row (cparts > 1) store the same value.
    float dm = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) dm = fmaxf(dm, sm.red[0][w]);
    a.errb[(int64_t)h * a.num_qblocks + gq] = kLn2 * __fsqrt_rn(qn2) * dm * (1.f + 0x1p-10f);
  }
}

template <int QDT>
hipError_t launch_scores_t(const ScoresArgs& a, dim3 grid, hipStream_t st) {
  static std::atomic<uint64_t> smem_set;
  const hipError_t e = set_smem_limit(smem_set, (const void*)scores_kernel<QDT>, kScoresSmem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((scores_kernel<QDT>), grid, dim3(64 * kWaves), kScoresSmem, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scores(const Geometry& g, const SeqMap& m, const void* q, const float* q_scale,
                         const u16* k_mean_bf16, const float* kres, const float* bnorm,
                         float* scores, hipStream_t st) {
  // A launch with at most 128 (kv head, query block) rows (small chunks)
  // splits each row's key tiles over floor(256 / rows) workgroups (at most
  // 16), so that every CU has work; whole prompts never split.
  const int64_t rows = (int64_t)g.lists * g.num_qblocks;
  const int cparts = 2 * rows > 256 ? 1 : (int)std::min<int64_t>(16, 256 / rows);
  const dim3 grid((unsigned)(rows * cparts));
  ScoresArgs a;
  a.cparts = cparts;
  a.m = m;
  a.q = q;
  a.q_scale = q_scale;
  a.kmean16 = k_mean_bf16;
  a.kres = kres;
  a.bnorm = bnorm;
  a.scores = scores;
  a.errb = scores + g.num_rows * (int64_t)g.max_blocks;
  a.num_blocks = g.num_blocks;
  a.num_qblocks = g.num_qblocks;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.group = g.lgroup;
  a.lists = g.lists;
  a.kvdiv = g.kvdiv;
  a.max_blocks = g.max_blocks;
  if (g.qk_dtype == FP_BF16) return launch_scores_t<FP_BF16>(a, grid, st);
  if (g.qk_dtype == FP_E4M3) return launch_scores_t<FP_E4M3>(a, grid, st);
  if (g.qk_dtype == FP_F32) return launch_scores_t<FP_F32>(a, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace fp
