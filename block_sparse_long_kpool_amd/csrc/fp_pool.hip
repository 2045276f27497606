// Block pooling: mean of K and V over each 128-token block of the paged
// cache (FlashPrefill summary "长上下文加速 28 倍", 3.1 key pooling; FlashPrefill
// V2 paper reading 4.1, the block means kbar_J / vbar_J), in float64.
// HBM-bound: every K/V element is read exactly once.
#include "fp_internal.hpp"

namespace fp {

// One workgroup: kboff / qboff of the sequence map (chunked scans).
__global__ __launch_bounds__(256) void plan_kernel(SeqMap m) { plan_offsets(m); }

hipError_t launch_plan(const SeqMap& m, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, m);
  return hipGetLastError();
}

// Load 8 consecutive elements of one token row as float.  fp32 inputs are
// rounded to bf16 first: that is the value every kernel of the library uses.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* v) {
  if constexpr (DT == FP_BF16) {
    const uint4 r = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(base) + elem);
    const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else if constexpr (DT == FP_E4M3) {
    const uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(base) + elem);
    const unsigned w[2] = {r.x, r.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = e4m3_to_f32((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    const float t[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)f32_to_bf16(t[i]);
  }
}

// grid (NK key blocks, Hkv, 2 = {K, V}); 256 threads = 16 token lanes x 16
// chunks of 8 head-dim elements.  Every key block of the cache is pooled,
// cached prefix included.  The sums run in float64: the at most 128 stored
// values of a block (bf16 or e4m3 codes, 8 and 4 significant bits) add up
// exactly unless their magnitudes span more than ~2^38, and the division by
// n_J rounds once, so the means are the exact block means to float64
// rounding.  Summation order is fixed (deterministic).  The discovery copy
// of each key mean is kbar_J * lscale (lscale = softmax_scale * log2(e)),
// rounded once to bf16: dot products with it are log2-domain logits.
template <int KDT, int VDT>
__global__ __launch_bounds__(256) void pool_kernel(
    SeqMap m, const int32_t* __restrict__ page_table, int max_pages, int page_size, int hkv,
    int64_t num_blocks, const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const float* __restrict__ k_scale, double lscale, double* __restrict__ k_mean,
    double* __restrict__ v_mean, u16* __restrict__ k_mean_bf16, float* __restrict__ kres,
    float* __restrict__ bnorm) {
  __shared__ double red[16][kHeadDim + 2];
  __shared__ double2 nred[kHeadDim / 64];
  const int gb = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int s = find_seq(m.kboff, m.num_seqs, gb);
  const int J = gb - m.kboff[s];
  const int len = (m.ctx ? m.ctx[s] : 0) + m.cu[s + 1] - m.cu[s];
  const int p0 = J * kBlock;
  const int nJ = min(kBlock, len - p0);
  const int chunk = threadIdx.x & 15;
  const int tl = threadIdx.x >> 4;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  const int32_t* prow = page_table + (int64_t)s * max_pages;
  auto row_elem = [&](int p, int page) {
    return (((int64_t)page * page_size + p % page_size) * hkv + h) * kHeadDim + chunk * 8;
  };
  if (nJ == kBlock) {
    // whole block: all eight page lookups, then all eight row loads in
    // flight at once (one at a time leaves HBM half idle); same summation
    // order as the general loop below
    int page[kBlock / 16];
#pragma unroll
    for (int it = 0; it < kBlock / 16; ++it) page[it] = prow[(p0 + tl + 16 * it) / page_size];
    float v[kBlock / 16][8];
#pragma unroll
    for (int it = 0; it < kBlock / 16; ++it) {
      const int64_t elem = row_elem(p0 + tl + 16 * it, page[it]);
      if (is_v) load8<VDT>(v_cache, elem, v[it]); else load8<KDT>(k_cache, elem, v[it]);
    }
#pragma unroll
    for (int it = 0; it < kBlock / 16; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (double)v[it][i];
  } else {
    for (int t = tl; t < nJ; t += 16) {
      const int p = p0 + t;
      float v[8];
      const int64_t elem = row_elem(p, prow[p / page_size]);
      if (is_v) load8<VDT>(v_cache, elem, v); else load8<KDT>(k_cache, elem, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (double)v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[tl][chunk * 8 + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int d = threadIdx.x;
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += red[r][d];
    // e4m3: the codes' sum times the head's scale (each code times the scale
    // is exact in float64, so this is the sum of the decoded keys)
    if (!is_v && KDT == FP_E4M3) sum *= (double)k_scale[h];
    const double mean = sum / (double)nJ;
    const int64_t o = ((int64_t)h * num_blocks + gb) * kHeadDim + d;
    if (is_v) {
      v_mean[o] = mean;
    } else {
      k_mean[o] = mean;
      // lscale * kbar rounded to bf16 (once, from float64) for the
      // discovery MFMA, and the squared norms of its rounding residual
      // (exact: the residual of a nearest rounding is representable) and
      // of the rounded value, summed over the 128 dims (two waves)
      const double ms = mean * lscale;
      const u16 hb = f64_to_bf16_bits(ms);
      k_mean_bf16[o] = hb;
      const double hv = (double)bf16_bits_to_f32(hb);
      const double r = ms - hv;
      const double r2 = wave_sum_d(r * r), h2 = wave_sum_d(hv * hv);
      if ((d & 63) == 0) nred[d >> 6] = make_double2(r2, h2);
    }
  }
  if (!is_v) {  // uniform per workgroup
    __syncthreads();
    if (threadIdx.x == 0) {
      const double r2 = nred[0].x + nred[1].x, h2 = nred[0].y + nred[1].y;
      // |s_J - bf16(s_J)|_2 + kAccumRel |bf16(s_J)|_2 with s_J = lscale *
      // kbar_J, rounded up to fp32 (the factor covers the float64 sums,
      // square roots and the final rounding; kAccumRel, twice the fp32
      // accumulation term, also covers the float64 rounding of the scaling)
      const double b = (sqrt(r2) + kAccumRel * sqrt(h2)) * (1.0 + 0x1p-40);
      kres[(int64_t)h * num_blocks + gb] = (float)b * (1.f + 0x1p-22f);
      bnorm[(int64_t)h * num_blocks + gb] = (float)sqrt(h2) * (1.f + 0x1p-22f);
    }
  }
}

hipError_t launch_pool(const Geometry& g, const SeqMap& m, const int32_t* page_table,
                       const void* k_cache, const void* v_cache, const float* k_scale,
                       double lscale, double* k_mean, double* v_mean, u16* k_mean_bf16,
                       float* kres, float* bnorm, hipStream_t st) {
  dim3 grid((unsigned)g.num_blocks, (unsigned)g.hkv, 2);
#define FP_POOL(KD, VD)                                                                       \
  hipLaunchKernelGGL((pool_kernel<KD, VD>), grid, dim3(256), 0, st, m, page_table,            \
                     g.max_pages, g.page_size, g.hkv, g.num_blocks, k_cache,                   \
                     v_cache, k_scale, lscale, k_mean, v_mean, k_mean_bf16, kres, bnorm)
  if (g.qk_dtype == FP_BF16 && g.v_dtype == FP_BF16) FP_POOL(FP_BF16, FP_BF16);
  else if (g.qk_dtype == FP_E4M3 && g.v_dtype == FP_BF16) FP_POOL(FP_E4M3, FP_BF16);
  else if (g.qk_dtype == FP_F32 && g.v_dtype == FP_F32) FP_POOL(FP_F32, FP_F32);
  else return hipErrorInvalidValue;
#undef FP_POOL
  return hipGetLastError();
}

}  // namespace fp
