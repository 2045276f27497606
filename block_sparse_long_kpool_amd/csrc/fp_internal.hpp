// Internal declarations shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int64_t num_blocks;  // N = sum_s n_s
  int max_blocks;      // n_max
  int64_t num_rows;    // Hkv * N
  int64_t total_tokens;  // T
  int qk_dtype, v_dtype, out_dtype;
  float softmax_scale;
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

// Locate global block gb: sequence s with boff[s] <= gb < boff[s+1].
__device__ __forceinline__ int find_seq(const int* __restrict__ boff, int num_seqs, int gb) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (boff[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
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

// Block offsets boff[num_seqs + 1] from cu_seqlens (prefix of ceil(len/128)).
hipError_t launch_plan(const int32_t* cu_seqlens, int num_seqs, int32_t* boff, hipStream_t st);

hipError_t launch_pool(const Geometry& g, const int32_t* cu, const int32_t* boff,
                       const int32_t* page_table, const void* k_cache, const void* v_cache,
                       const float* k_scale, float* k_mean, float* v_mean,
                       u16* k_mean_bf16, hipStream_t st);

hipError_t launch_scores(const Geometry& g, const int32_t* cu, const int32_t* boff,
                         const void* q, const float* q_scale, const u16* k_mean_bf16,
                         float* scores, hipStream_t st);

hipError_t launch_select(const Geometry& g, const int32_t* cu, const int32_t* boff,
                         const void* q, const float* q_scale, const float* k_mean,
                         const float* scores, float alpha, int n_sink, int n_local,
                         uint32_t* keep_bits, int32_t* counts, int32_t* row_ptr,
                         int32_t* col_idx, hipStream_t st);

hipError_t launch_attn_prep(const Geometry& g, const int32_t* cu, int32_t* boff,
                            const float* k_mean, const float* v_mean, u16* km16, u16* vm16,
                            hipStream_t st);

hipError_t launch_attn(const Geometry& g, const int32_t* cu, const int32_t* boff,
                       const int32_t* page_table, const void* q, const void* k_cache,
                       const void* v_cache, const float* q_scale, const float* k_scale,
                       const int32_t* row_ptr, const int32_t* col_idx, const u16* km16,
                       const u16* vm16, int correction, void* out, float* lse, hipStream_t st);

}  // namespace fp
