// Max-based dynamic threshold, forced sink/local blocks and index compaction
// (FlashPrefill summary "长上下文加速 28 倍", 3.2: keep J when its score reaches
// alpha times the row maximum over J <= I, plus the first 256 and the last
// 512 tokens as a safety net; 3.3: compact the kept blocks into a dense list
// so the attention loop walks only them).
//
// Three kernels:
//   decide  one workgroup (4 waves) per CSR row, heaviest rows first:
//           re-weight (subtract the row max of the log scores), threshold,
//           forced blocks -> keep bitmask + count.  Entries whose fast
//           (bf16) score lies within the row's guard of the threshold are
//           re-evaluated in float64 from q and k_mean by the whole
//           workgroup, with the row maximum re-evaluated the same way, so
//           that every decision matches exact arithmetic.
//   scan    one workgroup: exclusive prefix sum of the counts -> row_ptr.
//   compact one wave per row (kRowsPerWg rows per workgroup): wavefront
//           ballot + popcount prefix writes the kept block indices in
//           ascending order, never past the row's slot of row_ptr.
#include "fp_internal.hpp"

namespace fp {

namespace {

// Fast-path error budget (natural-log units).  The discovery logits use the
// pooled keys rounded to bf16; the scores pass bounds, per score row, how far
// that rounding and the fp32 accumulation of the dot products can move any
// entry from its exact value (E, stored after the scores).  The fp32
// statistics (logit scaling, exp2 / log2, sums over at most 2048 rows and the
// merges) add an absolute error below 1e-4 plus a relative one below 2^-19
// of the score's magnitude; kStatAbs / kStatRel allow several times that.
// An entry l and the row max lmax are therefore each within
// E + stat(l) of exact, stat(x) = kStatAbs + kStatRel |x|, and every entry
// within guard = 2 E + stat(l) + stat(lmax) of the threshold (and every
// candidate within the same guard of the row max) is re-evaluated in
// float64; all other decisions are certain.
constexpr float kStatAbs = 1e-3f;
constexpr float kStatRel = 0x1p-17f;
constexpr int kRowsPerWg = 4;

constexpr int kSelThreads = 256;
constexpr int kBatch = 8;  // pooled keys evaluated exactly per pass over a row's queries

__device__ __forceinline__ double bf16_lo(unsigned w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(unsigned w) { return (double)__uint_as_float(w & 0xFFFF0000u); }

// Head-dim elements 8c .. 8c+7 of the query row starting at element e0, as
// the values the path consumes (bf16 widened; e4m3 codes decoded, the head's
// scale applied later; fp32 rounded to bf16 first, as everywhere on this
// path), in float64.
template <int QDT>
__device__ __forceinline__ void q_chunk8(const void* q, int64_t e0, int c, double* v) {
  if constexpr (QDT == FP_BF16) {
    const uint4 w = reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(q) + e0)[c];
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else if constexpr (QDT == FP_E4M3) {
    const uint2 w = reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(q) + e0)[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (double)e4m3_to_f32(((e < 4 ? w.x : w.y) >> (8 * (e & 3))) & 0xFFu);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + e0) + 2 * c;
    const float4 a = p[0], b = p[1];
    const float t[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (double)(float)f32_to_bf16(t[e]);
  }
}

// Exact scores of nb <= kBatch pooled keys (float64 kbar rows staged in LDS
// at kbs[b * 128 ..]) for the rows of (h, block I), in one pass over the
// query rows: ex[b] = ln sum_r exp(x_rb - ref) + ref, x_rb = scale * q_r .
// kbar_b, all in float64.  Thread t takes rows t, t + 256, ...; each query row is read
// once for all nb keys (two accumulators per key).  Called uniformly by every
// thread; every thread returns the same ex[].
template <int QDT>
__device__ void exact_scores(const void* q, const float* q_scale, const double* kbs, int nb, int hq,
                             int group, int h, int64_t tok0, int nI, double scale, double ref,
                             double (*red)[kBatch], double* ex) {
  const int R = group * nI;
  double acc[kBatch];
#pragma unroll
  for (int b = 0; b < kBatch; ++b) acc[b] = 0.0;
  for (int r = threadIdx.x; r < R; r += kSelThreads) {
    const int hh = r / nI;
    const int t = r - hh * nI;
    const int hq_idx = h * group + hh;
    const int64_t e0 = ((tok0 + t) * hq + hq_idx) * (int64_t)kHeadDim;
    double d0[kBatch], d1[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) d0[b] = d1[b] = 0.0;
    // the staged keys are re-read every row (opaque offset), not kept live;
    // the chunk loop stays rolled (unrolling it, or keeping several rows per
    // thread in flight, measured slower: more registers, fewer waves)
    int koff = 0;
    asm volatile("" : "+v"(koff));
#pragma unroll 1
    for (int c = 0; c < kHeadDim / 8; ++c) {
      double v[8];
      q_chunk8<QDT>(q, e0, c, v);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (b < nb) {
          const double2* kp = reinterpret_cast<const double2*>(kbs + koff + b * kHeadDim + 8 * c);
          const double2 k0 = kp[0], k1 = kp[1], k2 = kp[2], k3 = kp[3];
          d0[b] = fma(v[0], k0.x, d0[b]);
          d1[b] = fma(v[1], k0.y, d1[b]);
          d0[b] = fma(v[2], k1.x, d0[b]);
          d1[b] = fma(v[3], k1.y, d1[b]);
          d0[b] = fma(v[4], k2.x, d0[b]);
          d1[b] = fma(v[5], k2.y, d1[b]);
          d0[b] = fma(v[6], k3.x, d0[b]);
          d1[b] = fma(v[7], k3.y, d1[b]);
        }
      }
    }
    const double sq = QDT == FP_E4M3 ? scale * (double)q_scale[hq_idx] : scale;
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (b < nb) acc[b] += exp(sq * (d0[b] + d1[b]) - ref);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    if (b < nb) {
      const double v = wave_sum_d(acc[b]);
      if (lane == 0) red[wave][b] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < kBatch; ++b) {
    if (b < nb) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < kSelThreads / 64; ++w) tot += red[w][b];
      ex[b] = log(tot) + ref;
    }
  }
  __syncthreads();  // red and the staged keys are reused by the next batch
}

// One workgroup per CSR row.  Pass 1 (threads over J, wave ballots): the fast
// keep bits and two candidate bitmaps in LDS, one for entries within the guard
// of the threshold (never forced blocks) and one for entries within the guard
// of the row max.  Pass 2, only if a threshold candidate exists: the max
// candidates and then the threshold candidates, in batches of kBatch keys
// evaluated exactly in one pass over the row's queries each; the exact row
// max is complete before the first threshold candidate is decided (the max
// candidates come first).  Pass 3 writes every word of the row's bitmask and
// the count.
template <int QDT>
__global__ __launch_bounds__(kSelThreads) void decide_kernel(
    SeqMap m, int hq, int kvdiv, int group, int64_t num_blocks, int64_t num_qblocks,
    int max_blocks, double softmax_scale,
    const void* __restrict__ q, const float* __restrict__ q_scale,
    const double* __restrict__ k_mean, const float* __restrict__ scores,
    const float* __restrict__ errb, float alpha, int n_sink,
    int n_local, uint32_t* __restrict__ keep_bits, int32_t* __restrict__ counts) {
  constexpr int kW = kMaxBlocksPerSeq / 32;
  __shared__ uint32_t keep_fast[kW + 1], cand_thr[kW + 1], cand_max[kW + 1], keep_fix[kW + 1];
  __shared__ float redf[kSelThreads / 64];
  __shared__ int redi[kSelThreads / 64];  // the waves' candidate flags
  // the waves' counts: a separate array, since without candidates no barrier
  // separates a wave's count from another wave still reading the flags
  __shared__ int redc[kSelThreads / 64];
  __shared__ double redd[kSelThreads / 64][kBatch];
  __shared__ __attribute__((aligned(16))) double kbs[kBatch * kHeadDim];
  __shared__ int bj[kBatch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // heaviest rows first: last query block first, the list owners interleaved
  // (a row's re-check work grows with its length; the long rows then do not
  // form the launch's tail)
  const int64_t lists = (int64_t)gridDim.x / num_qblocks;
  const int h = (int)((int64_t)blockIdx.x % lists);
  const int gq = (int)(num_qblocks - 1 - (int64_t)blockIdx.x / lists);
  const int64_t row = (int64_t)h * num_qblocks + gq;
  const QBlock qb = query_block(m, gq);
  const int I = qb.I;
  const int words = (max_blocks + 31) >> 5;
  uint32_t* bits = keep_bits + row * words;
  const float* L = scores + row * max_blocks;
  const int ncols = I + 1;
  const int nw_row = (ncols + 31) >> 5;

  if (!(alpha > 0.f)) {  // alpha <= 0 (or NaN): every causal block
    for (int w = tid; w < words; w += kSelThreads) {
      const int lo = 32 * w;
      bits[w] = lo >= ncols ? 0u : (ncols - lo >= 32 ? 0xFFFFFFFFu : ((1u << (ncols - lo)) - 1u));
    }
    if (tid == 0) counts[row] = ncols;
    return;
  }

  // row max of the fast log scores (re-weighting against the top block)
  float lmax = -INFINITY;
  for (int J = tid; J < ncols; J += kSelThreads) lmax = fmaxf(lmax, L[J]);
  lmax = wave_max(lmax);
  if (lane == 0) redf[wave] = lmax;
  __syncthreads();
  lmax = redf[0];
#pragma unroll
  for (int w = 1; w < kSelThreads / 64; ++w) lmax = fmaxf(lmax, redf[w]);
  const float lna = __logf(alpha);
  const float thr = lna + lmax;
  const float guard0 = 2.f * errb[row] + kStatAbs + kStatRel * fabsf(lmax);

  // pass 1: fast decisions and candidate bitmaps
  int need_l = 0;
  for (int base = 64 * wave; base < 32 * nw_row; base += kSelThreads) {
    const int J = base + lane;
    bool kp = false, ct = false, cm = false;
    if (J < ncols) {
      const float l = L[J];
      const bool forced = J < n_sink || I - J < n_local;
      const float guard = guard0 + kStatAbs + kStatRel * fabsf(l);
      kp = forced || l >= thr;
      ct = !forced && fabsf(l - thr) <= guard;
      cm = l >= lmax - guard;
    }
    const unsigned long long bk = __ballot(kp), bt = __ballot(ct), bm = __ballot(cm);
    need_l |= bt != 0ull;
    if (lane == 0) {
      const int w = base >> 5;  // w + 1 <= kW (the arrays hold kW + 1 words)
      keep_fast[w] = (uint32_t)bk;
      keep_fast[w + 1] = (uint32_t)(bk >> 32);
      cand_thr[w] = (uint32_t)bt;
      cand_thr[w + 1] = (uint32_t)(bt >> 32);
      cand_max[w] = (uint32_t)bm;
      cand_max[w + 1] = (uint32_t)(bm >> 32);
    }
  }
  if (lane == 0) redi[wave] = need_l;
  __syncthreads();
  int need = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) need |= redi[w];

  // pass 2: exact evaluation (uniform loops over the candidate bitmaps)
  if (need) {
    const int nI = qb.nI;
    const int64_t tok0 = qb.tok0;
    // list owner h: rows of its query heads h * group .. (group of them),
    // pooled keys of its KV head h / kvdiv
    const double* kb = k_mean + ((int64_t)(h / kvdiv) * num_blocks + qb.kb0) * kHeadDim;
    const double ref = (double)lmax;
    const double lnalpha = log((double)alpha);
    for (int w = tid; w < nw_row; w += kSelThreads) keep_fix[w] = 0u;
    double emax = -INFINITY;
    int nb = 0;
    uint32_t thr_mask = 0u;  // batch entries that are threshold candidates
    auto flush = [&]() {
      __syncthreads();  // bj[] written by thread 0; keep_fix cleared
      for (int e = tid; e < nb * kHeadDim; e += kSelThreads)
        kbs[e] = kb[(int64_t)bj[e / kHeadDim] * kHeadDim + e % kHeadDim];
      __syncthreads();
      double ex[kBatch];
      exact_scores<QDT>(q, q_scale, kbs, nb, hq, group, h, tok0, nI, softmax_scale, ref,
                        redd, ex);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (b < nb) {
          if (!((thr_mask >> b) & 1u)) {
            emax = fmax(emax, ex[b]);
          } else if (tid == 0 && ex[b] >= lnalpha + emax) {
            keep_fix[bj[b] >> 5] |= 1u << (bj[b] & 31);
          }
        }
      }
      __syncthreads();  // bj[] is rewritten by the next batch
      nb = 0;
      thr_mask = 0u;
    };
    for (int kind = 0; kind < 2; ++kind) {  // max candidates first, then threshold candidates
      for (int w = 0; w < nw_row; ++w) {
        uint32_t mw = kind == 0 ? cand_max[w] : cand_thr[w];
        while (mw) {
          const int b = __ffs(mw) - 1;
          mw &= mw - 1u;
          if (tid == 0) bj[nb] = 32 * w + b;
          if (kind) thr_mask |= 1u << nb;
          if (++nb == kBatch) flush();
        }
      }
    }
    if (nb) flush();
  }

  // pass 3: every word of the row (blocks past the diagonal are zero)
  int cnt = 0;
  for (int w = tid; w < words; w += kSelThreads) {
    uint32_t v = 0u;
    if (w < nw_row) {
      v = keep_fast[w];
      if (need) v = (v & ~cand_thr[w]) | keep_fix[w];
    }
    bits[w] = v;
    cnt += __popc(v);
  }
  cnt = (int)wave_sum((float)cnt);
  if (lane == 0) redc[wave] = cnt;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) tot += redc[w];
    counts[row] = tot;
  }
}

// Ranked selection: top-k / top-p, the prior methods' strategies that the
// FlashPrefill summary (section 二) contrasts with the max-based threshold
// and its ablation 4.4 compares against.  One workgroup per CSR row sorts the
// row's scores (bitonic sort in LDS, descending, ties toward the lower J: the
// key is the order-preserving image of the float above the complement of J)
// and keeps the forced blocks plus
//   top-k: the first k non-forced blocks of the ranking, or
//   top-p: the shortest ranked prefix (all causal blocks) whose share of
//          sum_J e^{L_IJ} reaches p (partial sums in a fixed order).
// The decisions use the scores as given (the fast fp32 path): entries within
// its error of the cut may rank differently from exact arithmetic.
constexpr int kRankThreads = 256;
struct RankSmem {
  unsigned long long key[kMaxBlocksPerSeq];
  uint32_t keep[kMaxBlocksPerSeq / 32];
  float part[kRankThreads];
  float off[kRankThreads];
  int cut;
};

template <int MODE>  // 0: top-k, 1: top-p
__global__ __launch_bounds__(kRankThreads) void rank_kernel(
    SeqMap m, int64_t num_qblocks, int max_blocks, const float* __restrict__ scores, int top_k,
    float top_p, int n_sink, int n_local, uint32_t* __restrict__ keep_bits,
    int32_t* __restrict__ counts) {
  extern __shared__ __attribute__((aligned(16))) char rank_smem[];
  RankSmem& sm = *reinterpret_cast<RankSmem*>(rank_smem);
  const int tid = threadIdx.x;
  // heaviest rows (longest sorts) first, as in the threshold selection
  const int64_t lists = (int64_t)gridDim.x / num_qblocks;
  const int gq = (int)(num_qblocks - 1 - (int64_t)blockIdx.x / lists);
  const int64_t row = ((int64_t)blockIdx.x % lists) * num_qblocks + gq;
  const QBlock qb = query_block(m, gq);
  const int I = qb.I;
  const int ncols = I + 1;
  int P = 1;
  while (P < ncols) P <<= 1;
  const float* L = scores + row * max_blocks;
  auto forced = [&](int J) { return J < n_sink || I - J < n_local; };
  const int words = (max_blocks + 31) >> 5;
  for (int i = tid; i < P; i += kRankThreads) {
    unsigned long long k = 0;  // padding and excluded entries sort last
    if (i < ncols && (MODE == 1 || !forced(i))) {
      uint32_t b = __float_as_uint(L[i]);
      b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
      k = ((unsigned long long)b << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
    }
    sm.key[i] = k;
  }
  for (int w = tid; w < words; w += kRankThreads) sm.keep[w] = 0u;
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kRankThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = sm.key[i], b = sm.key[ixj];
          if (((i & kk) == 0) ? (a < b) : (a > b)) {
            sm.key[i] = b;
            sm.key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  auto block_of = [&](int i) { return (int)(0xFFFFFFFFu - (uint32_t)(sm.key[i] & 0xFFFFFFFFull)); };
  int nkeep = 0;  // ranked entries kept: sorted positions 0 .. nkeep-1
  if constexpr (MODE == 0) {
    // forced blocks: the sinks J < n_sink and the window J > I - n_local
    const int nf = min(n_sink, ncols) + max(0, ncols - max(n_sink, I - n_local + 1));
    nkeep = min(max(top_k, 0), ncols - nf);
  } else {
    if (top_p > 0.f) {
      // thread t sums the sorted positions [t * seg, (t + 1) * seg)
      const int seg = (ncols + kRankThreads - 1) / kRankThreads;
      const float lmax = L[block_of(0)];
      const int i0 = tid * seg, i1 = min(ncols, i0 + seg);
      float acc = 0.f;
      for (int i = i0; i < i1; ++i) acc += __expf(L[block_of(i)] - lmax);
      sm.part[tid] = acc;
      if (tid == 0) sm.cut = ncols - 1;
      __syncthreads();
      if (tid == 0) {
        float run = 0.f;
        for (int t = 0; t < kRankThreads; ++t) {
          sm.off[t] = run;
          run += sm.part[t];
        }
        sm.part[0] = run;  // total (part[0] already consumed into off[1])
      }
      __syncthreads();
      const float target = top_p * sm.part[0];
      float cum = sm.off[tid];
      for (int i = i0; i < i1; ++i) {
        cum += __expf(L[block_of(i)] - lmax);
        if (cum >= target) {
          atomicMin(&sm.cut, i);
          break;
        }
      }
      __syncthreads();
      nkeep = sm.cut + 1;
    }
  }
  for (int i = tid; i < nkeep; i += kRankThreads) {
    const int J = block_of(i);
    atomicOr(&sm.keep[J >> 5], 1u << (J & 31));
  }
  for (int J = tid; J < ncols; J += kRankThreads)
    if (forced(J)) atomicOr(&sm.keep[J >> 5], 1u << (J & 31));
  __syncthreads();
  uint32_t* bits = keep_bits + row * words;
  int cnt = 0;
  for (int w = tid; w < words; w += kRankThreads) {
    const uint32_t v = sm.keep[w];
    bits[w] = v;
    cnt += __popc(v);
  }
  sm.part[tid] = (float)cnt;  // exact: counts are small integers
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int t = 0; t < kRankThreads; ++t) tot += (int)sm.part[t];
    counts[row] = tot;
  }
}

// Exclusive scan of counts[nrows] -> row_ptr[nrows + 1] (one workgroup).
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int64_t nrows, int32_t* __restrict__ row_ptr) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < nrows; base += 1024) {
    const int64_t i = base + tid;
    const int32_t v = i < nrows ? counts[i] : 0;
    int32_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int32_t w = lane < 16 ? wsum[lane] : 0;
      for (int o = 1; o < 16; o <<= 1) {
        const int32_t y = __shfl_up(w, o, 64);
        if (lane >= o) w += y;
      }
      if (lane < 16) wsum[lane] = w;
    }
    __syncthreads();
    const int32_t carry = carry_s;
    const int32_t excl = carry + (wave ? wsum[wave - 1] : 0) + x - v;
    if (i < nrows) row_ptr[i] = excl;
    __syncthreads();
    if (tid == 1023) carry_s = excl + v;
    __syncthreads();
  }
  if (tid == 0) row_ptr[nrows] = carry_s;
}

// kRowsPerWg rows per workgroup, one wave each.
__global__ __launch_bounds__(64 * kRowsPerWg) void compact_kernel(int64_t nrows, int max_blocks,
                                                      const uint32_t* __restrict__ keep_bits,
                                                      const int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int words = (max_blocks + 31) >> 5;
  const uint32_t* bits = keep_bits + row * words;
  int32_t* dst = col_idx + row_ptr[row];
  // the row's slot: never written past, whatever the bit row holds
  const int cap = row_ptr[row + 1] - row_ptr[row];
  int base_out = 0;
  for (int base = 0; base < 32 * words; base += 64) {
    const int w = base >> 5;
    const uint32_t lo = bits[w];
    const uint32_t hi = (w + 1 < words) ? bits[w + 1] : 0u;
    const unsigned long long m = ((unsigned long long)hi << 32) | lo;
    const bool keep = (m >> lane) & 1ull;
    const int pos = __popcll(m & ((1ull << lane) - 1ull));
    if (keep && base_out + pos < cap) dst[base_out + pos] = base + lane;
    base_out += __popcll(m);
  }
}

unsigned compact_grid(int64_t nrows) { return (unsigned)((nrows + kRowsPerWg - 1) / kRowsPerWg); }

}  // namespace

hipError_t launch_select_ranked(const Geometry& g, const SeqMap& m, const float* scores, int mode,
                                int top_k, float top_p, int n_sink, int n_local, uint32_t* keep_bits,
                                int32_t* counts, int32_t* row_ptr, int32_t* col_idx, hipStream_t st) {
  const unsigned nwg = (unsigned)g.num_rows;
  const size_t shm = sizeof(RankSmem);
  static std::atomic<uint64_t> smem_set[2];
  const void* fn = mode == 0 ? (const void*)rank_kernel<0> : (const void*)rank_kernel<1>;
  const hipError_t ea = set_smem_limit(smem_set[mode], fn, shm);
  if (ea != hipSuccess) return ea;
  if (mode == 0)
    hipLaunchKernelGGL(rank_kernel<0>, dim3(nwg), dim3(kRankThreads), shm, st, m, g.num_qblocks,
                       g.max_blocks, scores, top_k, top_p, n_sink, n_local, keep_bits, counts);
  else
    hipLaunchKernelGGL(rank_kernel<1>, dim3(nwg), dim3(kRankThreads), shm, st, m, g.num_qblocks,
                       g.max_blocks, scores, top_k, top_p, n_sink, n_local, keep_bits, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, g.num_rows, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, dim3(compact_grid(g.num_rows)), dim3(64 * kRowsPerWg), 0, st,
                     g.num_rows, g.max_blocks, keep_bits, row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_select(const Geometry& g, const SeqMap& m, const void* q, const float* q_scale,
                         const double* k_mean, const float* scores, float alpha, int n_sink,
                         int n_local, uint32_t* keep_bits, int32_t* counts, int32_t* row_ptr,
                         int32_t* col_idx, hipStream_t st) {
  const unsigned nwg = (unsigned)g.num_rows;
#define FP_DEC(QD)                                                                              \
  hipLaunchKernelGGL((decide_kernel<QD>), dim3(nwg), dim3(kSelThreads), 0, st, m, g.hq, g.kvdiv, \
                     g.lgroup, g.num_blocks, g.num_qblocks, g.max_blocks, g.softmax_scale_d, q,  \
                     q_scale, k_mean, scores, scores + g.num_rows * (int64_t)g.max_blocks, alpha, \
                     n_sink, n_local, keep_bits, counts)
  if (g.qk_dtype == FP_BF16) FP_DEC(FP_BF16);
  else if (g.qk_dtype == FP_E4M3) FP_DEC(FP_E4M3);
  else if (g.qk_dtype == FP_F32) FP_DEC(FP_F32);
  else return hipErrorInvalidValue;
#undef FP_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, g.num_rows, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, dim3(compact_grid(g.num_rows)), dim3(64 * kRowsPerWg), 0, st,
                     g.num_rows, g.max_blocks, keep_bits, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace fp
