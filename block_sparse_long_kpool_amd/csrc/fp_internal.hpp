// Internal declarations shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/flashprefill.h"

namespace fp {

constexpr int kBlock = 128;     // tokens per block (FlashPrefill V2 paper reading, section 四)
constexpr int kHeadDim = 128;
constexpr int kMaxBlocksPerSeq = 8192;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

// Host-side launch description shared by all kernels of one call.
struct Geometry {
  int num_seqs;
  int hq, hkv, group;
  int page_size, max_pages;
  int64_t num_blocks;    // NK = sum_s nk_s key blocks (pooled rows)
  int64_t num_qblocks;   // NQ = sum_s nq_s query blocks (score / CSR rows per KV head)
  int max_blocks;        // max_s nk_s
  int64_t num_rows;      // lists * NQ (score / CSR rows)
  int64_t csr_capacity;  // lists * causal blocks of the query blocks (<= INT32_MAX)
  // Index-list owners: the KV heads (lists = Hkv, lgroup = group query heads
  // per list, kvdiv = 1) or, per query head, lists = Hq, lgroup = 1 and
  // kvdiv = group (owner o reads KV head o / kvdiv).
  int lists, lgroup, kvdiv;
  int64_t total_tokens;  // T (query tokens)
  int qk_dtype, v_dtype, out_dtype;
  float softmax_scale;     // fp32 logit scale of the fast paths
  double softmax_scale_d;  // the same scale in float64 (1/sqrt(128) unrounded by
                           // default) for the exact re-evaluation
  int attn_splits;  // requested KV split of the attention (0: automatic)
};

// KV split of the attention: a launch with fewer (row, head-pack) workgroups
// than kAttnSplitTarget (one per CU) splits each row's tile list into
// floor(kAttnSplitTarget / workgroups) parts, at most kAttnMaxSplits, merged
// by a combine pass.  (Measured on 512- and 1K-token chunks after a 127K
// prefix: more parts than CUs only add partial-output traffic.)
constexpr int kAttnMaxSplits = 8;
constexpr int kAttnSplitTarget = 256;

// Where the tokens and blocks of each sequence live (device pointers).  The
// query tokens cu[s] .. cu[s+1]-1 are the positions ctx[s] .. ctx[s]+qlen-1
// of sequence s, whose KV cache holds klen = ctx[s] + qlen tokens (ctx is 0
// without a cached prefix, else a multiple of 128: chunked prefill).  Key
// block J < nk = ceil(klen / 128) is pooled row kboff[s] + J; the query
// blocks are I = ctx/128 .. nk-1, at rows qboff[s] + I - ctx/128.
struct SeqMap {
  const int32_t* cu;
  const int32_t* ctx;  // NULL: no cached prefix
  int32_t* kboff;      // [num_seqs + 1], written by launch_plan
  int32_t* qboff;      // [num_seqs + 1]
  int num_seqs;
};

// ---- device helpers -------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
  return __uint_as_float(((unsigned)b) << 16);
}

// OCP E4M3FN code -> float (exact): E = 0 is subnormal m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(unsigned c) {
  unsigned s = (c & 0x80u) << 24;
  unsigned e = (c >> 3) & 0xFu;
  unsigned m = c & 0x7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return __uint_as_float(__float_as_uint(mag) | s);
}

__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }

// float64 -> bf16 bits, rounded once to nearest even: truncate to fp32, set
// the fp32 sticky bit when that was inexact (round to odd), then round the
// fp32 value to nearest even (24 >= 8 + 2 bits, so the two steps equal one
// correct rounding).  Finite inputs.
__device__ __forceinline__ u16 f64_to_bf16_bits(double x) {
  const float t = __double2float_rz(x);
  const unsigned odd = (double)t != x ? 1u : 0u;
  const float f = __uint_as_float(__float_as_uint(t) | odd);
  return __builtin_bit_cast(u16, f32_to_bf16(f));
}

// Relative error allowance of a 128-term fp32 dot product of exactly
// representable products (MFMA with fp32 accumulation): n - 1 additions,
// each off by less than one ulp (2^-23, which covers truncating as well as
// nearest rounding), give less than 127 * 2^-23 < 2^-16 of the sum of the
// absolute products; kAccumRel doubles that.
constexpr double kAccumRel = 0x1p-15;

// Locate global block gb: sequence s with boff[s] <= gb < boff[s+1].
__device__ __forceinline__ int find_seq(const int* __restrict__ boff, int num_seqs, int gb) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (boff[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One query block (score / CSR row gq of a KV head): sequence, block index
// I inside the sequence, its query-token count and first query-token row,
// the sequence's key length and first pooled row.
struct QBlock {
  int s, I, nI, klen, kb0;
  int64_t tok0;
};
__device__ __forceinline__ QBlock query_block(const SeqMap& m, int gq) {
  QBlock r;
  r.s = find_seq(m.qboff, m.num_seqs, gq);
  const int c = m.ctx ? m.ctx[r.s] : 0;
  const int local = gq - m.qboff[r.s];
  r.I = c / kBlock + local;
  r.klen = c + (m.cu[r.s + 1] - m.cu[r.s]);
  r.nI = min(kBlock, r.klen - r.I * kBlock);
  r.tok0 = (int64_t)m.cu[r.s] + (int64_t)local * kBlock;
  r.kb0 = m.kboff[r.s];
  return r;
}

// The same block with every field in scalar registers (the values are
// wave-uniform; loaded through vector memory they would otherwise occupy
// VGPRs for the whole kernel).
__device__ __forceinline__ QBlock uniform_block(const QBlock& q) {
  QBlock r;
  r.s = __builtin_amdgcn_readfirstlane(q.s);
  r.I = __builtin_amdgcn_readfirstlane(q.I);
  r.nI = __builtin_amdgcn_readfirstlane(q.nI);
  r.klen = __builtin_amdgcn_readfirstlane(q.klen);
  r.kb0 = __builtin_amdgcn_readfirstlane(q.kb0);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)q.tok0);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)q.tok0 >> 32));
  r.tok0 = (int64_t)(((uint64_t)hi << 32) | lo);
  return r;
}

// Both block prefixes of SeqMap, by one workgroup of 256 threads.
__device__ __forceinline__ void plan_offsets(const SeqMap& m) {
  __shared__ int bufk[256], bufq[256];
  __shared__ int carry_k, carry_q;
  if (threadIdx.x == 0) carry_k = carry_q = 0;
  __syncthreads();
  for (int base = 0; base < m.num_seqs; base += 256) {
    const int s = base + (int)threadIdx.x;
    int nk = 0, nq = 0;
    if (s < m.num_seqs) {
      const int c = m.ctx ? m.ctx[s] : 0;
      nk = (c + m.cu[s + 1] - m.cu[s] + kBlock - 1) / kBlock;
      nq = nk - c / kBlock;
    }
    bufk[threadIdx.x] = nk;
    bufq[threadIdx.x] = nq;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int xk = (int)threadIdx.x >= o ? bufk[threadIdx.x - o] : 0;
      const int xq = (int)threadIdx.x >= o ? bufq[threadIdx.x - o] : 0;
      __syncthreads();
      bufk[threadIdx.x] += xk;
      bufq[threadIdx.x] += xq;
      __syncthreads();
    }
    const int ck = carry_k, cq = carry_q;
    if (s < m.num_seqs) {
      m.kboff[s] = ck + bufk[threadIdx.x] - nk;
      m.qboff[s] = cq + bufq[threadIdx.x] - nq;
    }
    __syncthreads();
    if (threadIdx.x == 255) {
      carry_k = ck + bufk[255];
      carry_q = cq + bufq[255];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    m.kboff[m.num_seqs] = carry_k;
    m.qboff[m.num_seqs] = carry_q;
  }
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- LDS staging ------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lds is wave-uniform and lane i's bytes land at lds + 16 i.  Completion is
// tracked by vmcnt only, so wait_vm() must precede the barrier that publishes
// the data.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void*)g, (lds_void*)lds, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Read through the constant address space: with a wave-uniform address this
// is a scalar load (tracked by lgkmcnt, so it does not wait behind vector
// loads in flight).  Only for data that no thread writes during the kernel.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// LDS has 64 banks of 4 bytes (256 bytes per row of banks).  Physical 16-byte
// chunk of logical chunk c in row r of a 256-byte bf16 row: c ^ g(r & 15),
// g swapping the two 2-bit halves of the row index.  Then (a) 16 consecutive
// rows read at one logical chunk (an MFMA operand gathered across rows) hit 16
// different chunks, and (b) 4 consecutive rows x 4 consecutive chunks (the
// V^T transposed reads of a 32-lane half) hit 16 different chunks: both
// patterns are conflict-free.  The map is an involution in c and depends on
// the row only through r & 15.
__device__ __forceinline__ int swz16(int c, int r) { return c ^ (((r & 3) << 2) | ((r >> 2) & 3)); }
// 128-byte fp8 rows (8 chunks, two rows per bank row): chunk c ^ ((r >> 1) & 7),
// again a function of r & 15 only.
__device__ __forceinline__ int swz8(int c, int r) { return c ^ ((r >> 1) & 7); }

// Sum / max of the value held by lanes l and l ^ 32 (v_permlane32_swap
// exchanges the two 32-lane halves; combining both outputs symmetrically gives
// the pair result in every lane).
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Issue order inside one pipeline block with NM MFMAs and ND LDS reads: each
// MFMA is preceded by its share of the LDS reads and followed by independent
// VALU work (the previous chunk's softmax), so the in-order wave keeps
// issuing VALU while the matrix core runs.
template <int NM, int ND>
__device__ __forceinline__ void interleave() {
  constexpr int kD = (ND + NM - 1) / NM;
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kD, 0);  // LDS reads run two MFMAs ahead
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
    __builtin_amdgcn_sched_group_barrier(0x100, kD, 0);  // DS read
  }
}

// ---- launchers (one per translation unit) ---------------------------------

// Raise a kernel's dynamic LDS limit to `bytes` once per device (bit d of
// `done` records device d; devices >= 64 are set on every launch).  Racing
// host threads may both set it, which is harmless: the call is idempotent.
inline hipError_t set_smem_limit(std::atomic<uint64_t>& done, const void* fn, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Block offsets kboff / qboff of the map (one workgroup).
hipError_t launch_plan(const SeqMap& m, hipStream_t st);

// Pooling (float64 means) also writes kbar rounded to bf16 and, per key
// block, the bound kres_J = |kbar_J - bf16(kbar_J)|_2 + kAccumRel
// |bf16(kbar_J)|_2 on how far a query row of unit norm can move its bf16 dot
// product with kbar_J from the exact one (rounding of kbar, plus fp32
// accumulation of 128 exact products).
hipError_t launch_pool(const Geometry& g, const SeqMap& m, const int32_t* page_table,
                       const void* k_cache, const void* v_cache, const float* k_scale,
                       double lscale, double* k_mean, double* v_mean, u16* k_mean_bf16,
                       float* kres, float* bnorm, hipStream_t st);

// Scores [lists * NQ, max_blocks] followed by one error bound per score row.
// bnorm: |bf16(kbar_J)|_2 per pooled key (rounded up), from the pooling pass.
hipError_t launch_scores(const Geometry& g, const SeqMap& m, const void* q, const float* q_scale,
                         const u16* k_mean_bf16, const float* kres, const float* bnorm,
                         float* scores, hipStream_t st);

hipError_t launch_select(const Geometry& g, const SeqMap& m, const void* q, const float* q_scale,
                         const double* k_mean, const float* scores, float alpha, int n_sink,
                         int n_local, uint32_t* keep_bits, int32_t* counts, int32_t* row_ptr,
                         int32_t* col_idx, hipStream_t st);

// Top-k (mode 0) / top-p (mode 1) selection from the scores, then the same
// scan and compaction as the threshold path.
hipError_t launch_select_ranked(const Geometry& g, const SeqMap& m, const float* scores, int mode,
                                int top_k, float top_p, int n_sink, int n_local, uint32_t* keep_bits,
                                int32_t* counts, int32_t* row_ptr, int32_t* col_idx, hipStream_t st);

// Block offsets of the map plus bf16 copies of the pooled keys / values.
hipError_t launch_attn_prep(const Geometry& g, const SeqMap& m, const double* k_mean,
                            const double* v_mean, u16* km16, u16* vm16, int* queue, hipStream_t st);

// Parts per row of the attention launch (1: no split).
int attn_splits(const Geometry& g);

// dense: every causal block of each row (no index lists, no correction;
// row_ptr / col_idx / km16 / vm16 unused).
hipError_t launch_attn(const Geometry& g, const SeqMap& m, const int32_t* page_table, const void* q,
                       const void* k_cache, const void* v_cache, const float* q_scale,
                       const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx,
                       const u16* km16, const u16* vm16, int correction, void* out, float* lse,
                       float* opart, float* lpart, int* queue, hipStream_t st,
                       bool dense);

}  // namespace fp
