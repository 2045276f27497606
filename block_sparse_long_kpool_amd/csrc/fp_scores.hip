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
// One workgroup (8 waves) owns one (h, I) and ALL its rows, so Q is read from
// HBM exactly once; the pooled keys of head h (bf16, L2-resident) stream
// through LDS in tiles of 64.  X = Q . Kbar^T runs on v_mfma_f32_32x32x16_bf16
// with A = Q (rows) and B = Kbar^T (pooled keys), the pooled keys split into
// two bf16 terms (hi + lo, two MFMAs into one fp32 accumulator) so the fast
// logits carry errors of a few 1e-5 only: in the result layout every
// lane owns one pooled-key column and 16 rows, so the per-column max and
// exp-sum are lane-local; lanes l and l^32 share a column and the 8 waves are
// merged through LDS.
#include "fp_internal.hpp"

namespace fp {

namespace {

constexpr int kWaves = 8;
constexpr int kJTile = 64;               // pooled keys per LDS tile
constexpr int kKbStride = kHeadDim + 8;  // bf16 elements per LDS row (272 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1e30f;

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

// RC = 32-row chunks per wave per pass; rows per pass = 8 waves * 32 * RC.
template <int QDT, int RC>
__global__ __launch_bounds__(512) void scores_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ boff, int num_seqs, int hq,
    int hkv, int group, int64_t num_blocks, int max_blocks, float logit_scale,
    const void* __restrict__ q, const float* __restrict__ q_scale,
    const u16* __restrict__ kmean16, float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) u16 kb[2][2][kJTile * kKbStride];  // [buf][hi/lo]
  __shared__ float2 part[2][kWaves][kJTile];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // heaviest rows (largest I) first
  const int64_t item = (int64_t)hkv * num_blocks - 1 - blockIdx.x;
  const int h = (int)(item % hkv);
  const int gb = (int)(item / hkv);
  const int s = find_seq(boff, num_seqs, gb);
  const int I = gb - boff[s];
  const int len = cu[s + 1] - cu[s];
  const int nI = min(kBlock, len - I * kBlock);
  const int64_t tok0 = (int64_t)cu[s] + (int64_t)I * kBlock;
  const u16* kbase = kmean16 + ((int64_t)h * num_blocks + boff[s]) * kHeadDim;
  const int64_t lo_off = (int64_t)hkv * num_blocks * kHeadDim;  // lo part follows the hi part
  float* out_row = scores + ((int64_t)h * num_blocks + gb) * max_blocks;
  const int ncols = I + 1;
  const int ntiles = (ncols + kJTile - 1) / kJTile;
  const int nchunks = 4 * group;  // 32-row chunks: (head, 32-token slice)
  constexpr int kChunksPerPass = kWaves * RC;

  for (int pass = 0; pass * kChunksPerPass < nchunks; ++pass) {
    // ---- Q fragments for this pass (read once) ----
    bf16x8 qf[RC][8];
    float cscale[RC];
    int nvalid[RC];
#pragma unroll
    for (int rc = 0; rc < RC; ++rc) {
      const int c = pass * kChunksPerPass + rc * kWaves + wave;
      const int hh = c >> 2;
      const int t0 = 32 * (c & 3);
      const bool head_ok = c < nchunks;
      nvalid[rc] = head_ok ? max(0, min(32, nI - t0)) : 0;
      const int hq_idx = h * group + (head_ok ? hh : 0);
      const bool rvalid = col < nvalid[rc];
      const int64_t row_elem = ((tok0 + t0 + col) * hq + hq_idx) * (int64_t)kHeadDim;
      load_q_frag<QDT>(q, row_elem, rvalid, half, qf[rc]);
      float sc = logit_scale * kLog2e;
      if constexpr (QDT == FP_E4M3) sc *= q_scale[hq_idx];
      cscale[rc] = sc;
    }

    // ---- stage pooled-key tile 0 (hi and lo parts) ----
    auto stage_load = [&](int tile, uint4* regs) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int c = it * 512 + (int)threadIdx.x;  // 16-byte chunk id in the tile
        const int r = c >> 4, part16 = c & 15;
        const int J = tile * kJTile + r;
        const u16* src = kbase + (int64_t)J * kHeadDim + part16 * 8;
        regs[it] = J < ncols ? *reinterpret_cast<const uint4*>(src) : uint4{0, 0, 0, 0};
        regs[2 + it] = J < ncols ? *reinterpret_cast<const uint4*>(src + lo_off) : uint4{0, 0, 0, 0};
      }
    };
    auto stage_store = [&](int buf, const uint4* regs) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int c = it * 512 + (int)threadIdx.x;
        const int r = c >> 4, part16 = c & 15;
        *reinterpret_cast<uint4*>(&kb[buf][0][r * kKbStride + part16 * 8]) = regs[it];
        *reinterpret_cast<uint4*>(&kb[buf][1][r * kKbStride + part16 * 8]) = regs[2 + it];
      }
    };
    {
      uint4 regs[4];
      stage_load(0, regs);
      stage_store(0, regs);
    }
    __syncthreads();

    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      uint4 nxt[4];
      const bool more = tile + 1 < ntiles;
      if (more) stage_load(tile + 1, nxt);

#pragma unroll
      for (int jc = 0; jc < kJTile / 32; ++jc) {
        const int boffs = (jc * 32 + col) * kKbStride + 64 * half;
        float m_l = kNegBig;
        f32x16 acc[RC];
#pragma unroll
        for (int rc = 0; rc < RC; ++rc) acc[rc] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&kb[buf][0][boffs + 8 * kk]);
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&kb[buf][1][boffs + 8 * kk]);
#pragma unroll
          for (int rc = 0; rc < RC; ++rc) {
            acc[rc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rc][kk], bh, acc[rc], 0, 0, 0);
            acc[rc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rc][kk], bl, acc[rc], 0, 0, 0);
          }
        }
#pragma unroll
        for (int rc = 0; rc < RC; ++rc) {
          // rows of this lane: m = 8*(i/4) + 4*half + (i%4)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * half + (i & 3);
            const float y = m < nvalid[rc] ? acc[rc][i] * cscale[rc] : -INFINITY;
            acc[rc][i] = y;
            m_l = fmaxf(m_l, y);
          }
        }
        float s_l = 0.f;
#pragma unroll
        for (int rc = 0; rc < RC; ++rc)
#pragma unroll
          for (int i = 0; i < 16; ++i) s_l += __builtin_amdgcn_exp2f(acc[rc][i] - m_l);
        const float m_p = __shfl_xor(m_l, 32, 64);
        const float s_p = __shfl_xor(s_l, 32, 64);
        const float m = fmaxf(m_l, m_p);
        const float s = s_l * __builtin_amdgcn_exp2f(m_l - m) + s_p * __builtin_amdgcn_exp2f(m_p - m);
        if (half == 0) part[buf][wave][jc * 32 + col] = make_float2(m, s);
      }

      if (more) stage_store(buf ^ 1, nxt);
      __syncthreads();

      if (threadIdx.x < kJTile) {
        const int J = tile * kJTile + (int)threadIdx.x;
        float m = kNegBig;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) m = fmaxf(m, part[buf][w][threadIdx.x].x);
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float2 p = part[buf][w][threadIdx.x];
          s += p.y * __builtin_amdgcn_exp2f(p.x - m);
        }
        if (J < ncols) {
          // log2 domain -> natural log; passes after the first merge with the
          // value already stored
          float L = (m + __log2f(s)) * kLn2;
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
}

}  // namespace

hipError_t launch_scores(const Geometry& g, const int32_t* cu, const int32_t* boff, const void* q,
                         const float* q_scale, const u16* k_mean_bf16, float* scores,
                         hipStream_t st) {
  const dim3 grid((unsigned)(g.hkv * g.num_blocks));
#define FP_SC(QD, RC)                                                                          \
  hipLaunchKernelGGL((scores_kernel<QD, RC>), grid, dim3(512), 0, st, cu, boff, g.num_seqs,    \
                     g.hq, g.hkv, g.group, g.num_blocks, g.max_blocks, g.softmax_scale, q,      \
                     q_scale, k_mean_bf16, scores)
#define FP_SC_RC(QD)                                  \
  do {                                                \
    if (g.group >= 8) FP_SC(QD, 4);                   \
    else if (g.group >= 4) FP_SC(QD, 2);              \
    else FP_SC(QD, 1);                                \
  } while (0)
  if (g.qk_dtype == FP_BF16) FP_SC_RC(FP_BF16);
  else if (g.qk_dtype == FP_E4M3) FP_SC_RC(FP_E4M3);
  else if (g.qk_dtype == FP_F32) FP_SC_RC(FP_F32);
  else return hipErrorInvalidValue;
#undef FP_SC_RC
#undef FP_SC
  return hipGetLastError();
}

}  // namespace fp
