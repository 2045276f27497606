// Sparse paged causal attention with block-mean correction.
//
// Method (FlashPrefill V2 paper reading): the attention stage walks only the
// compacted block list of each query block (FlashPrefill summary "长上下文加速
// 28 倍", 3.3) and folds, for every pruned block J, a pseudo-key with logit
// q . kbar_J + ln n_J and value vbar_J into the same softmax (4.1); the g
// query heads that share a KV head share each loaded K/V tile (PackGQA,
// 4.2(1)); K/V tiles are gathered straight from the paged cache through the
// page table (4.3).
//
// gfx950 design:
//   * workgroup = 4 waves = 256 query rows = 2 heads of one GQA group x the
//     128 tokens of one query block; wave w owns head 2*pack + w/2, tokens
//     64*(w%2) .. +63 as two 32-row chunks.  The g/2 workgroups of a group
//     are given consecutive ids on the same XCD so their K/V reads share L2.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (or the 32x32x64 OCP-fp8 MFMA
//     for e4m3 Q/K): A = K from LDS, B = Q^T held in registers for the whole
//     kernel.  In the result layout each lane owns one query row and 16 keys
//     per 32-key chunk, so the online softmax is lane-local plus one l^32
//     exchange.
//   * O^T = V^T P^T: B = P^T comes straight from the lane's own softmax
//     registers; A = V^T is read from the natural [key][d] LDS tile with
//     ds_read_b64_tr_b16 (16x4 transposes inside 16-lane groups).
//   * K/V tiles are double-buffered in LDS; the next tile's global loads are
//     issued before the current tile's math.
//   * correction tiles: 128 pooled keys/values (bf16) per tile with a
//     log2(n_J) bias; listed blocks and J > I are masked to -inf.
#include "fp_internal.hpp"

namespace fp {

namespace {

constexpr int kStride = kHeadDim + 8;       // bf16 elements per LDS row (272 B)
constexpr int kStride8 = kHeadDim + 16;     // bytes per LDS row of an fp8 K tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const int32_t* cu;
  const int32_t* boff;
  const int32_t* page_table;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* q_scale;
  const float* k_scale;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const u16* km16;
  const u16* vm16;
  void* out;
  float* lse;
  int64_t num_blocks;
  int64_t total_tokens;
  int num_seqs, max_pages, page_size;
  int hq, hkv, group, packs;
  int correction;
  float softmax_scale;
};

struct SharedMem {
  u16 k[2][kBlock * kStride];
  u16 v[2][kBlock * kStride];
  float bias[2][kBlock];
  uint32_t kept_bits[kMaxBlocksPerSeq / 32];
  int pooled_list[kMaxBlocksPerSeq / kBlock];
  int npooled;
};

__device__ __forceinline__ bf16x4 lds_read_tr(const u16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<u16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ uint2 f32x4_to_bf16x4(float4 a) {
  bf16x2 lo = bf16x2{f32_to_bf16(a.x), f32_to_bf16(a.y)};
  bf16x2 hi = bf16x2{f32_to_bf16(a.z), f32_to_bf16(a.w)};
  return uint2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Tile staging.  A tile is either a kept key block J of the sequence (gathered
// from the paged cache) or a pooled tile pt (bf16 kbar/vbar rows 128pt..+127).
// PREFETCH: global loads go to registers first (stage_load) and are written
// to LDS after the current tile's math (stage_store); fp32 caches are loaded
// and converted synchronously inside stage_store instead.
template <int QDT, int VDT>
struct Stager {
  static constexpr bool kPrefetch = QDT != FP_F32;
  uint4 kr[8];
  uint4 vr[8];

  __device__ __forceinline__ void load(const AttnArgs& a, int s, int h, int len, int64_t pooled_base,
                                       bool pooled, int idx, int I) {
    if constexpr (!kPrefetch) return;
    const int tid = threadIdx.x;
    if (pooled) {
      // only pooled rows J <= I exist for this query block
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int c = it * 256 + tid, key = c >> 4, part = c & 15;
        const int J = idx * kBlock + key;
        uint4 kx = uint4{0, 0, 0, 0}, vx = uint4{0, 0, 0, 0};
        if (J <= I) {
          const int64_t off = (pooled_base + J) * kHeadDim + part * 8;
          kx = *reinterpret_cast<const uint4*>(a.km16 + off);
          vx = *reinterpret_cast<const uint4*>(a.vm16 + off);
        }
        kr[it] = kx;
        vr[it] = vx;
      }
      return;
    }
    const int64_t ptrow = (int64_t)s * a.max_pages;
    // K
    if constexpr (QDT == FP_E4M3) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int c = it * 256 + tid, key = c >> 3, part = c & 7;
        const int p = idx * kBlock + key;
        uint4 r = uint4{0, 0, 0, 0};
        if (p < len) {
          const int page = a.page_table[ptrow + p / a.page_size];
          const int64_t e = (((int64_t)page * a.page_size + p % a.page_size) * a.hkv + h) * kHeadDim + part * 16;
          r = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.k_cache) + e);
        }
        kr[it] = r;
      }
    } else {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int c = it * 256 + tid, key = c >> 4, part = c & 15;
        const int p = idx * kBlock + key;
        uint4 r = uint4{0, 0, 0, 0};
        if (p < len) {
          const int page = a.page_table[ptrow + p / a.page_size];
          const int64_t e = (((int64_t)page * a.page_size + p % a.page_size) * a.hkv + h) * kHeadDim + part * 8;
          r = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(a.k_cache) + e);
        }
        kr[it] = r;
      }
    }
    // V (bf16)
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = it * 256 + tid, key = c >> 4, part = c & 15;
      const int p = idx * kBlock + key;
      uint4 r = uint4{0, 0, 0, 0};
      if (p < len) {
        const int page = a.page_table[ptrow + p / a.page_size];
        const int64_t e = (((int64_t)page * a.page_size + p % a.page_size) * a.hkv + h) * kHeadDim + part * 8;
        r = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(a.v_cache) + e);
      }
      vr[it] = r;
    }
  }

  __device__ __forceinline__ void store(const AttnArgs& a, SharedMem& sm, int buf, int s, int h,
                                        int len, int64_t pooled_base, bool pooled, int idx, int I) {
    const int tid = threadIdx.x;
    if (pooled && tid < kBlock) {
      const int J = idx * kBlock + tid;
      const bool kept = (sm.kept_bits[J >> 5] >> (J & 31)) & 1u;
      const int nJ = min(kBlock, len - J * kBlock);
      sm.bias[buf][tid] = (J <= I && !kept) ? __log2f((float)nJ) : -INFINITY;
    }
    if constexpr (kPrefetch) {
      if (pooled || QDT == FP_BF16) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int c = it * 256 + tid, key = c >> 4, part = c & 15;
          *reinterpret_cast<uint4*>(&sm.k[buf][key * kStride + part * 8]) = kr[it];
        }
      } else {
        uint8_t* kb = reinterpret_cast<uint8_t*>(sm.k[buf]);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int c = it * 256 + tid, key = c >> 3, part = c & 7;
          *reinterpret_cast<uint4*>(kb + key * kStride8 + part * 16) = kr[it];
        }
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int c = it * 256 + tid, key = c >> 4, part = c & 15;
        *reinterpret_cast<uint4*>(&sm.v[buf][key * kStride + part * 8]) = vr[it];
      }
    } else {
      // fp32 caches (and their pooled tiles): load, round to bf16, store.
      const int64_t ptrow = (int64_t)s * a.max_pages;
      for (int it = 0; it < 16; ++it) {
        const int c = it * 256 + tid, key = c >> 5, part = c & 31;
        uint2 kw = uint2{0, 0}, vw = uint2{0, 0};
        if (pooled) {
          const int J = idx * kBlock + key;
          if (J <= I) {
            const int64_t off = (pooled_base + J) * kHeadDim + part * 4;
            kw = *reinterpret_cast<const uint2*>(a.km16 + off);
            vw = *reinterpret_cast<const uint2*>(a.vm16 + off);
          }
        } else {
          const int p = idx * kBlock + key;
          if (p < len) {
            const int page = a.page_table[ptrow + p / a.page_size];
            const int64_t e = (((int64_t)page * a.page_size + p % a.page_size) * a.hkv + h) * kHeadDim + part * 4;
            kw = f32x4_to_bf16x4(*reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.k_cache) + e));
            vw = f32x4_to_bf16x4(*reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.v_cache) + e));
          }
        }
        *reinterpret_cast<uint2*>(&sm.k[buf][key * kStride + part * 4]) = kw;
        *reinterpret_cast<uint2*>(&sm.v[buf][key * kStride + part * 4]) = vw;
      }
    }
  }
};

template <int QDT, int VDT, int ODT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SharedMem& sm = *reinterpret_cast<SharedMem*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work item: XCD-grouped (row, pack), heaviest rows first ----
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int kq = b >> 3;
  const int pack = kq % a.packs;
  const int64_t row_ord = (int64_t)(kq / a.packs) * 8 + xcd;
  const int64_t nrows = (int64_t)a.hkv * a.num_blocks;
  if (row_ord >= nrows) return;
  const int h = (int)(row_ord % a.hkv);
  const int gb = (int)(a.num_blocks - 1 - row_ord / a.hkv);
  const int64_t row = (int64_t)h * a.num_blocks + gb;
  const int s = find_seq(a.boff, a.num_seqs, gb);
  const int I = gb - a.boff[s];
  const int len = a.cu[s + 1] - a.cu[s];
  const int nI = min(kBlock, len - I * kBlock);
  const int64_t tok0 = (int64_t)a.cu[s] + (int64_t)I * kBlock;
  const int64_t pooled_base = (int64_t)h * a.num_blocks + a.boff[s];
  const int kbeg = a.row_ptr[row];
  const int nkept = a.row_ptr[row + 1] - kbeg;

  const int hh = 2 * pack + (wave >> 1);
  const bool head_ok = hh < a.group;
  const int hq_idx = h * a.group + (head_ok ? hh : 0);
  const int tbase = 64 * (wave & 1);

  // ---- kept-block bitmap and the pooled tiles that hold a pruned block ----
  const int nwords = (I >> 5) + 1;
  if (a.correction) {
    for (int w = tid; w < nwords; w += 256) sm.kept_bits[w] = 0u;
    __syncthreads();
    for (int i = tid; i < nkept; i += 256) {
      const int J = a.col_idx[kbeg + i];
      if ((unsigned)J <= (unsigned)I) atomicOr(&sm.kept_bits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    if (wave == 0) {
      const int ntile_p = (I >> 7) + 1;
      int cnt = 0;
      for (int base = 0; base < ntile_p; base += 64) {
        const int pt = base + lane;
        bool any_pruned = false;
        if (pt < ntile_p) {
          const int lo = pt * kBlock, hi = min(pt * kBlock + kBlock - 1, I);
          for (int w = lo >> 5; w <= (hi >> 5); ++w) {
            uint32_t m = ~sm.kept_bits[w];
            const int wlo = w * 32;
            if (wlo < lo) m &= ~((1u << (lo - wlo)) - 1u);
            if (wlo + 31 > hi) m &= (hi - wlo >= 31) ? 0xFFFFFFFFu : ((1u << (hi - wlo + 1)) - 1u);
            any_pruned |= m != 0u;
          }
        }
        const unsigned long long mb = __ballot(any_pruned);
        if (any_pruned) sm.pooled_list[cnt + __popcll(mb & ((1ull << lane) - 1ull))] = pt;
        cnt += __popcll(mb);
      }
      if (lane == 0) sm.npooled = cnt;
    }
    __syncthreads();
  }
  const int npooled = a.correction ? sm.npooled : 0;
  const int ntiles = nkept + npooled;

  // ---- Q^T fragments (B operand), kept for the whole kernel ----
  // lane owns row col of chunk rc; head-dim slots 64*half + 8*kk + i
  constexpr bool kFp8 = QDT == FP_E4M3;
  bf16x8 qf[2][8];
  i32x8 qf8[2][2];
  int nvalid[2];
#pragma unroll
  for (int rc = 0; rc < 2; ++rc) {
    const int t0 = tbase + 32 * rc;
    nvalid[rc] = head_ok ? max(0, min(32, nI - t0)) : 0;
    const bool rvalid = col < nvalid[rc];
    const int64_t e0 = ((tok0 + t0 + col) * a.hq + hq_idx) * (int64_t)kHeadDim + 64 * half;
    if constexpr (kFp8) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        i32x8 v = i32x8{};
        if (rvalid) {
          const i32x4* p = reinterpret_cast<const i32x4*>(reinterpret_cast<const uint8_t*>(a.q) + e0 + 32 * k2);
          const i32x4 lo = p[0], hi = p[1];
          v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        qf8[rc][k2] = v;
      }
      // bf16 copy for the pooled (correction) tiles: exact widening
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int k2 = kk >> 2, w0 = 2 * (kk & 3);
        const unsigned wlo = (unsigned)qf8[rc][k2][w0], whi = (unsigned)qf8[rc][k2][w0 + 1];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          qf[rc][kk][i] = f32_to_bf16(e4m3_to_f32(((i < 4 ? wlo : whi) >> (8 * (i & 3))) & 0xFFu));
      }
    } else if constexpr (QDT == FP_BF16) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qf[rc][kk] = rvalid ? *reinterpret_cast<const bf16x8*>(reinterpret_cast<const u16*>(a.q) + e0 + 8 * kk)
                            : bf16x8{};
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (rvalid) {
          const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q) + e0 + 8 * kk);
          const float4 x = p[0], y = p[1];
          qf[rc][kk] = bf16x8{f32_to_bf16(x.x), f32_to_bf16(x.y), f32_to_bf16(x.z), f32_to_bf16(x.w),
                              f32_to_bf16(y.x), f32_to_bf16(y.y), f32_to_bf16(y.z), f32_to_bf16(y.w)};
        } else {
          qf[rc][kk] = bf16x8{};
        }
      }
    }
  }
  // log2-domain logit scales: kept tiles and pooled tiles
  float c_kept = a.softmax_scale * kLog2e;
  float c_pool = c_kept;
  if constexpr (kFp8) {
    const float qs = a.q_scale[hq_idx];
    c_kept *= qs * a.k_scale[h];
    c_pool *= qs;
  }

  // ---- online-softmax state ----
  f32x16 o[2][4];
  float m_run[2], l_run[2];
#pragma unroll
  for (int rc = 0; rc < 2; ++rc) {
    m_run[rc] = -INFINITY;
    l_run[rc] = 0.f;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) o[rc][dc] = f32x16{};
  }

  auto tile_desc = [&](int t, bool& pooled) -> int {
    pooled = t >= nkept;
    return pooled ? sm.pooled_list[t - nkept] : a.col_idx[kbeg + t];
  };

  Stager<QDT, VDT> stg;
  if (ntiles > 0) {
    bool pooled;
    const int idx = tile_desc(0, pooled);
    stg.load(a, s, h, len, pooled_base, pooled, idx, I);
    stg.store(a, sm, 0, s, h, len, pooled_base, pooled, idx, I);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    bool pooled;
    const int idx = tile_desc(t, pooled);
    bool pooled_n = false;
    int idx_n = 0;
    const bool more = t + 1 < ntiles;
    if (more) {
      idx_n = tile_desc(t + 1, pooled_n);
      stg.load(a, s, h, len, pooled_base, pooled_n, idx_n, I);
    }

    // ---- S^T = K Q^T ----
    f32x16 sacc[2][4];
#pragma unroll
    for (int rc = 0; rc < 2; ++rc)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) sacc[rc][kc] = f32x16{};
    if (kFp8 && !pooled) {
      const uint8_t* kb = reinterpret_cast<const uint8_t*>(sm.k[buf]);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const i32x4* p = reinterpret_cast<const i32x4*>(kb + (kc * 32 + col) * kStride8 + 64 * half + 32 * k2);
          const i32x4 lo = p[0], hi = p[1];
          const i32x8 av = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rc = 0; rc < 2; ++rc)
            sacc[rc][kc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, qf8[rc][k2], sacc[rc][kc], 0, 0, 0, 127, 0, 127);
        }
      }
    } else {
      const u16* kb = sm.k[buf];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(kb + (kc * 32 + col) * kStride + 64 * half + 8 * kk);
#pragma unroll
          for (int rc = 0; rc < 2; ++rc)
            sacc[rc][kc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[rc][kk], sacc[rc][kc], 0, 0, 0);
        }
      }
    }

    // ---- online softmax (log2 domain) ----
    const float cs = pooled ? c_pool : c_kept;
    const bool diag = !pooled && idx == I;
    bf16x8 pb[2][8];
#pragma unroll
    for (int rc = 0; rc < 2; ++rc) {
      const int p_local = tbase + 32 * rc + col;
      float mloc = -INFINITY;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kc + 8 * (i >> 2) + 4 * half + (i & 3);
          float y = sacc[rc][kc][i] * cs;
          if (pooled) y += sm.bias[buf][key];
          if (diag && key > p_local) y = -INFINITY;
          sacc[rc][kc][i] = y;
          mloc = fmaxf(mloc, y);
        }
      }
      const float mnew = fmaxf(m_run[rc], fmaxf(mloc, __shfl_xor(mloc, 32, 64)));
      const float corr = __builtin_amdgcn_exp2f(m_run[rc] - mnew);
      m_run[rc] = mnew;
      float lsum = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pe = __builtin_amdgcn_exp2f(sacc[rc][kc][i] - mnew);
          lsum += pe;
          pb[rc][2 * kc + (i >> 3)][i & 7] = f32_to_bf16(pe);
        }
      }
      l_run[rc] = l_run[rc] * corr + lsum;
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) o[rc][dc] *= corr;
    }

    // ---- O^T += V^T P^T ----
    {
      const u16* vb = sm.v[buf];
      const int vrow = 4 * half + ((lane & 15) >> 2);
      const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const u16* p = vb + (16 * ks + vrow) * kStride + 32 * dc + vcol;
          const bf16x4 lo = lds_read_tr(p);
          const bf16x4 hi = lds_read_tr(p + 8 * kStride);
          const bf16x8 av = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rc = 0; rc < 2; ++rc)
            o[rc][dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[rc][ks], o[rc][dc], 0, 0, 0);
        }
      }
    }

    if (more) stg.store(a, sm, buf ^ 1, s, h, len, pooled_base, pooled_n, idx_n, I);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = m + log2(l) (natural log out) ----
#pragma unroll
  for (int rc = 0; rc < 2; ++rc) {
    const float l_tot = l_run[rc] + __shfl_xor(l_run[rc], 32, 64);
    const float inv = 1.f / l_tot;
    if (col >= nvalid[rc]) continue;
    const int64_t tok = tok0 + tbase + 32 * rc + col;
    const int64_t obase = (tok * a.hq + hq_idx) * (int64_t)kHeadDim;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dc + 8 * j + 4 * half;
        const float x0 = o[rc][dc][4 * j] * inv, x1 = o[rc][dc][4 * j + 1] * inv;
        const float x2 = o[rc][dc][4 * j + 2] * inv, x3 = o[rc][dc][4 * j + 3] * inv;
        if constexpr (ODT == FP_BF16) {
          *reinterpret_cast<uint2*>(reinterpret_cast<u16*>(a.out) + obase + d) =
              f32x4_to_bf16x4(make_float4(x0, x1, x2, x3));
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + obase + d) = make_float4(x0, x1, x2, x3);
        }
      }
    }
    if (a.lse && half == 0) a.lse[(int64_t)hq_idx * a.total_tokens + tok] = (m_run[rc] + __log2f(l_tot)) * kLn2;
  }
}

// boff (block 0 of the grid) and bf16 copies of the pooled keys / values.
__global__ __launch_bounds__(256) void attn_prep_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                        int32_t* __restrict__ boff, const float* __restrict__ km,
                                                        const float* __restrict__ vm, u16* __restrict__ km16,
                                                        u16* __restrict__ vm16, int64_t n) {
  if (blockIdx.x == gridDim.x - 1) {
    // sequential-in-chunks scan of ceil(len/128): one block
    __shared__ int buf[256];
    __shared__ int carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < num_seqs; base += 256) {
      const int s = base + (int)threadIdx.x;
      const int v = s < num_seqs ? (cu[s + 1] - cu[s] + kBlock - 1) / kBlock : 0;
      buf[threadIdx.x] = v;
      __syncthreads();
      for (int o = 1; o < 256; o <<= 1) {
        const int x = (int)threadIdx.x >= o ? buf[threadIdx.x - o] : 0;
        __syncthreads();
        buf[threadIdx.x] += x;
        __syncthreads();
      }
      const int c = carry;
      if (s < num_seqs) boff[s] = c + buf[threadIdx.x] - v;
      __syncthreads();
      if (threadIdx.x == 255) carry = c + buf[255];
      __syncthreads();
    }
    if (threadIdx.x == 0) boff[num_seqs] = carry;
    return;
  }
  if (km == nullptr) return;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 x = *reinterpret_cast<const float4*>(km + i);
  const float4 y = *reinterpret_cast<const float4*>(vm + i);
  *reinterpret_cast<uint2*>(km16 + i) = f32x4_to_bf16x4(x);
  *reinterpret_cast<uint2*>(vm16 + i) = f32x4_to_bf16x4(y);
}

}  // namespace

hipError_t launch_attn_prep(const Geometry& g, const int32_t* cu, int32_t* boff, const float* k_mean,
                            const float* v_mean, u16* km16, u16* vm16, hipStream_t st) {
  const int64_t n = (int64_t)g.hkv * g.num_blocks * kHeadDim;
  const unsigned conv = k_mean ? (unsigned)((n / 4 + 255) / 256) : 0u;
  hipLaunchKernelGGL(attn_prep_kernel, dim3(conv + 1), dim3(256), 0, st, cu, g.num_seqs, boff, k_mean,
                     v_mean, km16, vm16, n);
  return hipGetLastError();
}

hipError_t launch_attn(const Geometry& g, const int32_t* cu, const int32_t* boff, const int32_t* page_table,
                       const void* q, const void* k_cache, const void* v_cache, const float* q_scale,
                       const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx, const u16* km16,
                       const u16* vm16, int correction, void* out, float* lse, hipStream_t st) {
  AttnArgs a;
  a.cu = cu;
  a.boff = boff;
  a.page_table = page_table;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.km16 = km16;
  a.vm16 = vm16;
  a.out = out;
  a.lse = lse;
  a.num_blocks = g.num_blocks;
  a.num_seqs = g.num_seqs;
  a.max_pages = g.max_pages;
  a.page_size = g.page_size;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.group = g.group;
  a.packs = (g.group + 1) / 2;
  a.correction = correction;
  a.softmax_scale = g.softmax_scale;
  a.total_tokens = g.total_tokens;
  const int64_t rows = (int64_t)g.hkv * g.num_blocks;
  const unsigned grid = (unsigned)(((rows + 7) / 8) * 8 * a.packs);
  const size_t shm = sizeof(SharedMem);
#define FP_ATTN(QD, VD, OD)                                                                    \
  do {                                                                                         \
    static bool attr_set = false;                                                              \
    if (!attr_set) {                                                                           \
      hipError_t e = hipFuncSetAttribute((const void*)attn_kernel<QD, VD, OD>,                 \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm); \
      if (e != hipSuccess) return e;                                                           \
      attr_set = true;                                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((attn_kernel<QD, VD, OD>), dim3(grid), dim3(256), shm, st, a);          \
  } while (0)
#define FP_ATTN_O(QD, VD)                                  \
  do {                                                     \
    if (g.out_dtype == FP_BF16) FP_ATTN(QD, VD, FP_BF16);  \
    else FP_ATTN(QD, VD, FP_F32);                          \
  } while (0)
  if (g.qk_dtype == FP_BF16 && g.v_dtype == FP_BF16) FP_ATTN_O(FP_BF16, FP_BF16);
  else if (g.qk_dtype == FP_E4M3 && g.v_dtype == FP_BF16) FP_ATTN_O(FP_E4M3, FP_BF16);
  else if (g.qk_dtype == FP_F32 && g.v_dtype == FP_F32) FP_ATTN_O(FP_F32, FP_F32);
  else return hipErrorInvalidValue;
#undef FP_ATTN_O
#undef FP_ATTN
  return hipGetLastError();
}

}  // namespace fp
