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
//   * workgroup = 256 query rows = 2 heads of one GQA group x the 128 tokens
//     of one query block, split over 8 waves (two per SIMD, one 32-row chunk
//     each).  The g/2 workgroups of a group get ids 8 apart, i.e. the same
//     XCD at about the same time, so their K/V reads share that L2; the last
//     7 % of the items are handed out on demand so that the XCDs finish
//     together.
//   * K/V tiles move HBM -> LDS with global_load_lds_dwordx4 (no staging
//     registers): every lane gathers 16 bytes of a token row through the page
//     table and the hardware writes lane i's bytes at LDS base + 16 i.  Rows
//     are unpadded and 16-byte chunks are XOR-swizzled by row (swz16 /
//     swz8), which makes the MFMA operand reads below conflict-free.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (the OCP-fp8 32x32x64 MFMA for
//     e4m3 Q/K): A = K from LDS, B = Q^T held in registers for the whole
//     kernel.  In the result layout each lane owns one query row and 16 keys
//     per 32-key chunk, so the online softmax is lane-local plus one l^32
//     exchange; the running max is only raised when it grows by more than
//     64 (log2 units), so tiles almost never rescale the output accumulator.
//   * O^T = V^T P^T: B = P^T comes straight from the lane's own softmax
//     registers; A = V^T is read from the natural [key][d] LDS tile with
//     ds_read_b64_tr_b16 (16x4 transposes inside 16-lane groups).
//   * correction tiles: 128 pooled keys/values (bf16) per tile with a
//     log2(n_J) bias, which seeds the S^T accumulator (stored divided by
//     the head's logit scale, so the softmax is that of a kept tile);
//     listed blocks and J > I are masked to -inf the same way.
//   * rows: query blocks of the call (a chunk's blocks after a cached prefix,
//     or whole prompts); keys are every cached position up to the row.
//   * KV split (small launches): a row's tile list is cut into contiguous
//     parts, one workgroup each; parts write fp32 partial outputs and lse,
//     merged by attn_combine_kernel.
#include <algorithm>
#include <type_traits>

#include "fp_internal.hpp"

namespace fp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Tolerated growth of the running max (log2 units) before the output
// accumulator is rescaled.  Probabilities are formed as 2^(y - m) with a max m
// that may lag the true one by up to kLazy, i.e. values up to 2^64: far inside
// the bf16 / fp32 exponent range, and relative precision does not depend on
// magnitude.  In practice the rescale then runs at most once per row.
constexpr float kLazy = 64.0f;
constexpr float kLazyBound = 18446744073709551616.0f;  // 2^kLazy
// Initial running max: finite, so that a masked logit (-inf) minus it stays
// -inf (probability 0) and no inf - inf ever forms; any real logit exceeds it
// by far more than kLazy, so a row's first chunk always takes the exact path
// (its sum is +inf).  A row that has seen only masked keys keeps m = kMInit
// and l = 0.  (A part of a KV-split row may start with a diagonal or a
// correction tile, whose first chunk can be fully masked for some rows.)
constexpr float kMInit = -1e30f;
constexpr int kTileElems = kBlock * kHeadDim;  // one bf16 tile = 32 KiB
// waves per workgroup: two waves per SIMD, 32 query rows each (a form with
// four waves of 64 rows needs more than 512 registers per wave and spills)
constexpr int kAttnWaves = 8;
// On-demand tail of the item order (launches of at least kAttnDynMinItems
// items): its share of the items and the extra workgroups, in percent of it.
constexpr int64_t kAttnDynMinItems = 4096;
constexpr int64_t kAttnDynFracPct = 7;
constexpr int64_t kAttnDynSlackPct = 50;

struct AttnArgs {
  SeqMap m;
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
  float* opart;  // splits > 1: [splits, T, Hq, d] partial outputs (each normalised by its own sum)
  float* lpart;  // splits > 1: [splits, Hq, T] partial lse (natural log; -inf for an empty part)
  int splits;    // workgroups per (row, head pack), each over a contiguous part of the tile list
  int nitems;    // work items: rows (rounded up to 8) x packs x splits
  int dyn_begin; // items from here on are handed out through *queue (see the kernel)
  int* queue;    // counter of the dynamic items, zero at launch
  int64_t num_blocks;   // NK (pooled rows per KV head)
  int64_t num_qblocks;  // NQ (CSR rows per list owner)
  int64_t total_tokens;
  int max_pages, page_size;
  int hq, hkv, group, packs;  // group: query heads per index list (1 per query head)
  int lists, kvdiv;           // list owners; owner o reads KV head o / kvdiv
  int correction;
  float softmax_scale;
};

struct SharedMem {
  u16 k[2][kTileElems];  // fp8 tiles use the first half of a buffer
  u16 v[2][kTileElems];
  float bias[2][2][kBlock];  // [buffer][head slot]: log2(n_J) / c_pool or -inf
  // element offset ((page * page_size + offset) * Hkv + h) * d of each token
  // row of a kept tile in the paged K/V caches
  int64_t slot[2][kBlock];
  uint32_t kept_bits[kMaxBlocksPerSeq / 32];
  // tile list of the row: kept blocks (list order), then pooled tile indices
  uint16_t tiles[kMaxBlocksPerSeq + kMaxBlocksPerSeq / kBlock];
  int npooled;
  int item;  // a dynamic workgroup's item (-1: none left)
};

__device__ __forceinline__ bf16x4 lds_read_tr(const u16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(const_cast<u16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

// In-place rescale of an output accumulator (runs only when a row's running
// max grows by more than kLazy).
__device__ __forceinline__ void scale_acc(f32x16& x, float c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] *= c;
}

__device__ __forceinline__ uint2 f32x4_to_bf16x4(float4 a) {
  bf16x2 lo = bf16x2{f32_to_bf16(a.x), f32_to_bf16(a.y)};
  bf16x2 hi = bf16x2{f32_to_bf16(a.z), f32_to_bf16(a.w)};
  return uint2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// DENSE: every causal block 0..I of the row, in order, without index lists
// or correction (the dense causal baseline on the same kernel).
template <int QDT, int VDT, int ODT, int NW, bool DENSE>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnArgs a) {
  static_assert(NW == kAttnWaves, "one 32-row chunk per wave");
  constexpr int RC = 8 / NW;   // 32-row chunks per wave (the workgroup always covers 256 rows)
  constexpr int NT = 64 * NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SharedMem& sm = *reinterpret_cast<SharedMem*>(smem_raw);
  constexpr bool kFp8 = QDT == FP_E4M3;
  constexpr bool kF32 = QDT == FP_F32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work item: XCD-grouped (row, pack), heaviest rows first ----
  // Workgroups are dispatched to the eight XCDs in turn, so workgroup b runs
  // on XCD b % 8 and item b with it: the packs of a row (items 8 apart) run
  // together on one XCD and share its L2.  The XCDs do not all run at the
  // same speed, though, so the last items (dyn_begin on) are handed out on
  // demand instead: the workgroups from dyn_begin on (the grid has some
  // beyond nitems) take the next one from a counter, and a workgroup that
  // finds none left exits.  XCDs that are ahead thus take more of them.
  int b = blockIdx.x;
  if (b >= a.dyn_begin) {
    if (tid == 0) {
      const int j = atomicAdd(a.queue, 1);
      sm.item = j < a.nitems - a.dyn_begin ? a.dyn_begin + j : -1;
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(sm.item);
    if (b < 0) return;
  }
  const int xcd = b & 7;
  const int kq = b >> 3;
  const int pack = kq % a.packs;
  const int split = (kq / a.packs) % a.splits;
  const int64_t row_ord = (int64_t)(kq / a.packs / a.splits) * 8 + xcd;
  const int64_t nrows = (int64_t)a.lists * a.num_qblocks;
  if (row_ord >= nrows) return;
  const int h = (int)(row_ord % a.lists);  // list owner (CSR row h * NQ + gq)
  const int gq = (int)(a.num_qblocks - 1 - row_ord / a.lists);
  const int64_t row = (int64_t)h * a.num_qblocks + gq;
  // wave-uniform by construction; said explicitly so that the list bounds
  // below become scalar loads
  const int32_t* row_bounds = a.row_ptr + (int64_t)__builtin_amdgcn_readfirstlane((int)row);
  const int kvh = h / a.kvdiv;  // KV head of the owner's keys, values and pooled blocks
  const QBlock qb = uniform_block(query_block(a.m, gq));
  const int s = qb.s;
  const int I = qb.I;
  const int len = qb.klen;  // keys: cached prefix + this chunk
  const int nI = qb.nI;
  const int64_t tok0 = qb.tok0;
  const int64_t pooled_base = (int64_t)kvh * a.num_blocks + qb.kb0;
  // The row's list is the head of a chain of dependent loads (list -> page
  // table -> K/V gather), so it is read before anything else: its bounds by
  // scalar loads, the first NT entries into registers ahead of the Q loads
  // (a wait for them then does not wait for Q).
  const int kbeg = DENSE ? 0 : load_uniform(row_bounds);
  // a valid list holds at most I + 1 blocks (the LDS tile list is sized for it)
  const int nkept = DENSE ? I + 1 : min(max(load_uniform(row_bounds + 1) - kbeg, 0), I + 1);
  // entry min(tid, nkept - 1); an empty list reads its own bound instead
  // (branch-free, so that nothing waits for this load before the Q loads)
  const int first_entry =
      DENSE ? 0 : *(nkept > 0 ? a.col_idx + kbeg + min(tid, nkept - 1) : row_bounds);
  const int64_t ptrow = (int64_t)s * a.max_pages;

  const int hh = 2 * pack + (wave * RC) / 4;
  const bool head_ok = hh < a.group;
  const int hq_idx = __builtin_amdgcn_readfirstlane(h * a.group + (head_ok ? hh : 0));  // wave-uniform
  // 32-token slice of the wave.  Waves w and w + 4 share a SIMD; in the
  // sparse instance they take complementary slices (s and 3 - s) so that
  // every SIMD has the same causal work in the diagonal tile, whose chunks
  // past a wave's last row are skipped (the dense instance, where the
  // diagonal tile is one of many, keeps slice w % 4).
  const int slice = DENSE ? wave % 4 : (wave < 4 ? wave : 7 - wave);
  const int tbase = 32 * slice;

  // ---- Q^T fragments (B operand), kept for the whole kernel ----
  // (issued right after the list: their latency overlaps the list set-up
  // below).  Every lane loads unconditionally, rows past the block re-reading
  // its last token, and invalid rows are zeroed afterwards: without a branch
  // around the loads, a wait for the list loads issued before them does not
  // have to wait for these.
  // lane owns row col of chunk rc; head-dim slots 64*half + 8*kk + i
  bf16x8 qf[RC][8];
  i32x8 qf8[RC][2];
  int nvalid[RC];
#pragma unroll
  for (int rc = 0; rc < RC; ++rc) {
    const int t0 = tbase + 32 * rc;
    nvalid[rc] = __builtin_amdgcn_readfirstlane(head_ok ? max(0, min(32, nI - t0)) : 0);  // wave-uniform
    const bool rvalid = col < nvalid[rc];
    const int64_t e0 = ((tok0 + min(t0 + col, nI - 1)) * a.hq + hq_idx) * (int64_t)kHeadDim + 64 * half;
    if constexpr (kFp8) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const i32x4* p = reinterpret_cast<const i32x4*>(reinterpret_cast<const uint8_t*>(a.q) + e0 + 32 * k2);
        const i32x4 lo = p[0], hi = p[1];
        const i32x8 v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        qf8[rc][k2] = rvalid ? v : i32x8{};
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qf[rc][kk] = bf16x8{};
    } else if constexpr (QDT == FP_BF16) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const u16*>(a.q) + e0 + 8 * kk);
        qf[rc][kk] = rvalid ? v : bf16x8{};
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q) + e0 + 8 * kk);
        const float4 x = p[0], y = p[1];
        const bf16x8 v = bf16x8{f32_to_bf16(x.x), f32_to_bf16(x.y), f32_to_bf16(x.z), f32_to_bf16(x.w),
                                f32_to_bf16(y.x), f32_to_bf16(y.y), f32_to_bf16(y.z), f32_to_bf16(y.w)};
        qf[rc][kk] = rvalid ? v : bf16x8{};
      }
    }
  }
  // ---- tile list in LDS, kept-block bitmap, pooled tiles ----
  // The row's list is copied once so that every per-tile lookup is an LDS
  // read.  Entries are clamped to [0, I] for addressing (a list from the
  // selection stage is always in range; out-of-range entries from other
  // producers give unspecified output but no out-of-bounds access).
  const int nwords = (I >> 5) + 1;
  if (!DENSE && a.correction)
    for (int w = tid; w < nwords; w += NT) sm.kept_bits[w] = 0u;
  if (!DENSE) {
    if (tid < nkept) sm.tiles[tid] = (uint16_t)min(max(first_entry, 0), I);
    for (int i = tid + NT; i < nkept; i += NT) sm.tiles[i] = (uint16_t)min(max(a.col_idx[kbeg + i], 0), I);
  }
  __syncthreads();

  // Tile range of this workgroup.  Without a KV split it is the whole list
  // (kept tiles first): the first tile is then known before the pooled tiles
  // are counted, and its page lookups and gathers are issued here, ahead of
  // the bitmap and the scan below (tend is provisional until the scan).
  const bool early = a.splits == 1 && nkept > 0;
  int tbeg = 0;
  int tend = nkept;

  // log2-domain logit scales: kept tiles and pooled tiles
  float c_kept = a.softmax_scale * kLog2e;
  float c_pool = c_kept;
  if constexpr (kFp8) {
    const float qs = a.q_scale[hq_idx];
    c_kept *= qs * a.k_scale[kvh];
    c_pool *= qs;
  }
  // pooled-tile bias writers: thread t < 256 writes slot t / 128, whose head
  // may differ from its own wave's; the bias is stored divided by that
  // head's c_pool so that it can seed the MFMA accumulator
  float c_pool_w = a.softmax_scale * kLog2e;
  if constexpr (kFp8) {
    const int hh_w = 2 * pack + (tid >> 7);
    c_pool_w *= a.q_scale[h * a.group + (hh_w < a.group ? hh_w : 0)];
  }
  const int bslot = (wave * RC) / 4;  // this wave's head slot

  // ---- tile staging -------------------------------------------------------
  // Kept block J: token rows J*128 .. +127 of the sequence (rows past the end
  // of the sequence re-read the block's first token: finite values that the
  // causal mask removes).  Pooled tile pt: pooled rows pt*128 .. +127 of the
  // sequence (rows past I re-read row I; their bias is -inf).
  //
  // Page-table lookups run one tile ahead of the K/V gathers: threads 0..127
  // fetch the page of row `tid` of tile t+2 while tile t is computed and
  // publish the cache slot in sm.slot, so the gathers of tile t+1 never wait
  // on a dependent load.  Page sizes that divide 128 are powers of two
  // (shift / mask); larger ones are multiples of 128 (one page per block).
  const int psz = a.page_size;
  const bool small_pages = psz <= kBlock;
  const int pshift = 31 - __clz(psz);
  auto tile_index = [&](int t) { return DENSE ? t : (int)sm.tiles[t]; };
  // page id of row `tid` of kept tile t (only threads < 128); -1 if pooled
  auto fetch_page = [&](int t) -> int {
    if (t >= tend || t >= nkept || tid >= kBlock) return -1;
    const int J = tile_index(t);
    const int p0 = J * kBlock + tid;
    const int p = p0 < len ? p0 : J * kBlock;
    return a.page_table[ptrow + (small_pages ? (p >> pshift) : (p / psz))];
  };
  auto publish_slot = [&](int t, int page, int sbuf) {
    if (t >= tend || t >= nkept || tid >= kBlock) return;
    const int J = tile_index(t);
    const int p0 = J * kBlock + tid;
    const int p = p0 < len ? p0 : J * kBlock;
    const int cslot = page * psz + (small_pages ? (p & (psz - 1)) : (p % psz));
    sm.slot[sbuf][tid] = ((int64_t)cslot * a.hkv + kvh) * kHeadDim;
  };
  // slots of the first two tiles of the range (both page lookups in flight
  // together), published by the caller's next barrier
  auto prologue_slots = [&]() {
    const int page0 = fetch_page(tbeg);
    const int page1 = fetch_page(tbeg + 1);
    publish_slot(tbeg, page0, tbeg & 1);
    publish_slot(tbeg + 1, page1, (tbeg + 1) & 1);
  };
  auto issue_tile = [&](int t, int buf) {
    const bool pooled = t >= nkept;
    const int idx = tile_index(t);
    if (pooled && tid < 2 * kBlock) {
      const int j = tid & (kBlock - 1);
      const int J = idx * kBlock + j;
      const bool kept = (sm.kept_bits[J >> 5] >> (J & 31)) & 1u;
      const int nJ = min(kBlock, len - J * kBlock);
      sm.bias[buf][tid >> 7][j] = (J <= I && !kept) ? __log2f((float)nJ) / c_pool_w : -INFINITY;
    }
    const int64_t* slots = sm.slot[buf];
    if constexpr (kF32) {
      // fp32 cache: load, round to bf16, store swizzled (no async path)
      for (int it = 0; it < 2048 / NT; ++it) {
        const int c16 = it * NT + tid;  // 16-byte chunk of the bf16 tile
        const int r = c16 >> 4, c = c16 & 15;
        uint4 kw, vw;
        if (pooled) {
          const int J = min(idx * kBlock + r, I);
          kw = *reinterpret_cast<const uint4*>(a.km16 + (pooled_base + J) * kHeadDim + c * 8);
          vw = *reinterpret_cast<const uint4*>(a.vm16 + (pooled_base + J) * kHeadDim + c * 8);
        } else {
          const int64_t e = slots[r] + c * 8;
          const float* ks = reinterpret_cast<const float*>(a.k_cache) + e;
          const float* vs = reinterpret_cast<const float*>(a.v_cache) + e;
          const uint2 ka = f32x4_to_bf16x4(*reinterpret_cast<const float4*>(ks));
          const uint2 kb = f32x4_to_bf16x4(*reinterpret_cast<const float4*>(ks + 4));
          const uint2 va = f32x4_to_bf16x4(*reinterpret_cast<const float4*>(vs));
          const uint2 vb = f32x4_to_bf16x4(*reinterpret_cast<const float4*>(vs + 4));
          kw = uint4{ka.x, ka.y, kb.x, kb.y};
          vw = uint4{va.x, va.y, vb.x, vb.y};
        }
        const int off = r * kHeadDim + swz16(c, r) * 8;
        *reinterpret_cast<uint4*>(&sm.k[buf][off]) = kw;
        *reinterpret_cast<uint4*>(&sm.v[buf][off]) = vw;
      }
      return;
    }
    // bf16 rows: each wave-instruction fills 1 KiB = 4 rows of 256 B
    const int sub = lane >> 4, pc = lane & 15;
    if (pooled) {
#pragma unroll
      for (int it = 0; it < 32 / NW; ++it) {
        const int wi = wave * (32 / NW) + it;  // wave-instruction index: 1 KiB of the tile
        const int r = wi * 4 + sub;
        const int c = swz16(pc, r);
        const int J = min(idx * kBlock + r, I);
        const int64_t e = (pooled_base + J) * kHeadDim + c * 8;
        load_lds16(a.km16 + e, &sm.k[buf][wi * 512]);
        load_lds16(a.vm16 + e, &sm.v[buf][wi * 512]);
      }
      return;
    }
    const u16* vc = reinterpret_cast<const u16*>(a.v_cache);
    // all row offsets first (one LDS wait), then the gathers
    int64_t rowoff[32 / NW];
#pragma unroll
    for (int it = 0; it < 32 / NW; ++it) rowoff[it] = slots[(wave * (32 / NW) + it) * 4 + sub];
#pragma unroll
    for (int it = 0; it < 32 / NW; ++it) {
      const int wi = wave * (32 / NW) + it;
      const int r = wi * 4 + sub;
      const int64_t e = rowoff[it] + swz16(pc, r) * 8;
      load_lds16(vc + e, &sm.v[buf][wi * 512]);
      if constexpr (!kFp8) {
        load_lds16(reinterpret_cast<const u16*>(a.k_cache) + e, &sm.k[buf][wi * 512]);
      }
    }
    if constexpr (kFp8) {
      // fp8 rows of 128 B: each wave-instruction fills 8 rows
      const int sub8 = lane >> 3, pc8 = lane & 7;
      uint8_t* kb = reinterpret_cast<uint8_t*>(sm.k[buf]);
      int64_t rowoff8[16 / NW];
#pragma unroll
      for (int it = 0; it < 16 / NW; ++it) rowoff8[it] = slots[(wave * (16 / NW) + it) * 8 + sub8];
#pragma unroll
      for (int it = 0; it < 16 / NW; ++it) {
        const int wi = wave * (16 / NW) + it;
        const int r = wi * 8 + sub8;
        load_lds16(reinterpret_cast<const uint8_t*>(a.k_cache) + rowoff8[it] + swz8(pc8, r) * 16, kb + wi * 1024);
      }
    }
  };

  if (early) {
    prologue_slots();
    __syncthreads();
    issue_tile(0, 0);  // a kept tile: needs neither the bitmap nor the pooled list
  }

  if (!DENSE && a.correction) {
    for (int i = tid; i < nkept; i += NT) {
      const int J = sm.tiles[i];
      atomicOr(&sm.kept_bits[J >> 5], 1u << (J & 31));
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
        if (any_pruned) sm.tiles[nkept + cnt + __popcll(mb & ((1ull << lane) - 1ull))] = (uint16_t)pt;
        cnt += __popcll(mb);
      }
      if (lane == 0) sm.npooled = cnt;
    }
    __syncthreads();
  }
  // wave-uniform counts: keep them in scalar registers
  const int npooled = (!DENSE && a.correction) ? __builtin_amdgcn_readfirstlane(sm.npooled) : 0;
  const int ntiles = nkept + npooled;
  // KV split: this workgroup takes tiles [tbeg, tend) of the row's list
  // (contiguous parts balanced by tile count; all of it without a split)
  tbeg = (int)(((int64_t)split * ntiles) / a.splits);
  tend = (int)(((int64_t)(split + 1) * ntiles) / a.splits);

  // ---- online-softmax state ----
  f32x16 o[RC][4];
  float m_run[RC], l_run[RC];
#pragma unroll
  for (int rc = 0; rc < RC; ++rc) {
    m_run[rc] = kMInit;
    l_run[rc] = 0.f;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) o[rc][dc] = f32x16{};
  }

  // prologue: slots of the first two tiles, gathers of the first (already in
  // flight on the early path)
  if (!early) {
    prologue_slots();
    __syncthreads();
    if (tbeg < tend) issue_tile(tbeg, tbeg & 1);
  }
  wait_vm();
  __syncthreads();

  // Per-lane LDS offsets inside a tile.  Every operand read below touches a
  // row whose low four bits are fixed per lane (the key column for K, vrow and
  // vrow + 8 for V), so the row swizzle is loop-invariant: a read is a per-lane
  // base plus uniform offsets (half-tile, chunk row group), the latter folded
  // into the instruction's immediate.
  int koff[8];  // bf16 K: row col, logical chunk 8 half + kk (elements)
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = col * kHeadDim + swz16(8 * half + kk, col) * 8;
  int koff8[4];  // fp8 K: row col, logical 16-byte chunks 4 half + 0..3 (bytes)
#pragma unroll
  for (int c = 0; c < 4; ++c) koff8[c] = col * 128 + swz8(4 * half + c, col) * 16;
  // V^T transposed reads: 16-row groups, lane rows vrow and vrow + 8 of each
  const int vrow = 4 * half + ((lane & 15) >> 2);
  const int csel = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vsub = 4 * (lane & 1);
  int voff[4][2];
#pragma unroll
  for (int dc = 0; dc < 4; ++dc) {
    voff[dc][0] = vrow * kHeadDim + swz16(4 * dc + csel, vrow) * 8 + vsub;
    voff[dc][1] = (vrow + 8) * kHeadDim + swz16(4 * dc + csel, vrow + 8) * 8 + vsub;
  }

  // Kept tiles first, then pooled (correction) tiles: two loops over one
  // iteration body so each loop holds only the Q form it multiplies with
  // (fp8 codes for kept tiles of fp8 inputs, bf16 otherwise).
  auto iterate = [&](int t, auto pooled_c, auto diag_c) {
    constexpr bool POOLED_TILE = decltype(pooled_c)::value;
    const int buf = t & 1;
    if (t + 1 < tend) issue_tile(t + 1, buf ^ 1);
    const int page_next = fetch_page(t + 2);  // consumed after the math below

    // The 128-key tile runs as four 32-key chunks c in a software pipeline:
    // block c issues the MFMAs of S(c+1) = K Q^T and O += V P(c-1) together
    // with the online softmax of chunk c (VALU), which depends on neither, so
    // one wave keeps the matrix core and the VALU busy at once.  The lazy-max
    // rescale (rare) runs between blocks, after P(c-1) has been accumulated
    // relative to the previous max.  Kept / diagonal / pooled variants are
    // compile-time, so the softmax carries no per-element selects.
    constexpr bool POOLED = POOLED_TILE;
    constexpr bool DIAG = decltype(diag_c)::value;
    constexpr bool kQk8 = kFp8 && !POOLED;
    const u16* kt = sm.k[buf];
    const u16* vt = sm.v[buf];

    // S^T for keys 32 c .. +31: lane's query row col, keys 32 c + 8 (i/4) +
    // 4 half + i%4 in slot i
    auto qk = [&](int c, f32x16* sc) {
#pragma unroll
      for (int rc = 0; rc < RC; ++rc) {
        if constexpr (POOLED) {
          // the accumulator starts at the pooled keys' bias (in logit units)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const float4 bv = *reinterpret_cast<const float4*>(&sm.bias[buf][bslot][32 * c + 8 * jq + 4 * half]);
            sc[rc][4 * jq + 0] = bv.x;
            sc[rc][4 * jq + 1] = bv.y;
            sc[rc][4 * jq + 2] = bv.z;
            sc[rc][4 * jq + 3] = bv.w;
          }
        } else {
          sc[rc] = f32x16{};
        }
      }
      if constexpr (kQk8) {
        const uint8_t* kb = reinterpret_cast<const uint8_t*>(kt) + c * 32 * 128;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(kb + koff8[2 * k2]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(kb + koff8[2 * k2 + 1]);
          const i32x8 av = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rc = 0; rc < RC; ++rc)
            sc[rc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qf8[rc][k2], sc[rc], 0, 0, 0, 127, 0, 127);
        }
      } else {
        const u16* kb = kt + c * 32 * kHeadDim;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(kb + koff[kk]);
#pragma unroll
          for (int rc = 0; rc < RC; ++rc)
            sc[rc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[rc][kk], sc[rc], 0, 0, 0);
        }
      }
    };

    // O^T += V^T P^T over keys 32 c .. +31 (two 16-key MFMA steps)
    auto pv = [&](int c, const bf16x8 (*pp)[2]) {
      const u16* vb = vt + c * 32 * kHeadDim;
#pragma unroll
      for (int s16 = 0; s16 < 2; ++s16) {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) {
          const bf16x4 lo = lds_read_tr(vb + s16 * 16 * kHeadDim + voff[dc][0]);
          const bf16x4 hi = lds_read_tr(vb + s16 * 16 * kHeadDim + voff[dc][1]);
          const bf16x8 av = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rc = 0; rc < RC; ++rc)
            o[rc][dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pp[rc][s16], o[rc][dc], 0, 0, 0);
        }
      }
    };

    // Online softmax of chunk c (log2 domain) -> bf16 probabilities in the
    // P^T operand layout and the chunk's row sums.  Fast path: exponentiate
    // against the running max m_run as is.  The max only has to move when a
    // logit exceeds m_run + kLazy, and then that row's chunk sum exceeds
    // 2^kLazy (a row's first chunk, with m_run = kMInit, gives +inf), so the sum
    // doubles as the overflow test and the fast path computes no max at all.
    // The slow path (rare) raises the max of the affected rows, rescales the
    // output and recomputes the chunk.
    auto finish_logits = [&](int c, f32x16* sc) {
#pragma unroll
      for (int rc = 0; rc < RC; ++rc) {
        if constexpr (DIAG) {
          const int p_local = tbase + 32 * rc + col;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * c + 8 * (i >> 2) + 4 * half + (i & 3);
            if (key > p_local) sc[rc][i] = -INFINITY;
          }
        }
      }
    };
    auto exponentiate = [&](const f32x16* sc, bf16x8 (*pp)[2], float* ls) {
#pragma unroll
      for (int rc = 0; rc < RC; ++rc) {
        const float m = m_run[rc];
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float arg = fmaf(sc[rc][i], POOLED ? c_pool : c_kept, -m);
          const float pe = __builtin_amdgcn_exp2f(arg);
          lsum += pe;
          pp[rc][i >> 3][i & 7] = f32_to_bf16(pe);
        }
        ls[rc] = lsum;
      }
    };
    auto softmax = [&](int c, f32x16* sc, bf16x8 (*pp)[2], float* ls) -> bool {
      finish_logits(c, sc);
      exponentiate(sc, pp, ls);
      bool over = false;
#pragma unroll
      for (int rc = 0; rc < RC; ++rc) over |= !(ls[rc] <= kLazyBound);
      return over;
    };
    // The probabilities and row sums of the block are pinned before the
    // branch so that they stay inside the pipeline block (otherwise they are
    // sunk past it, next to their first use).
    auto settle = [&](bool over, f32x16* sc, bf16x8 (*pp)[2], float* ls) {
#pragma unroll
      for (int rc = 0; rc < RC; ++rc) asm volatile("" ::"v"(pp[rc][0]), "v"(pp[rc][1]), "v"(ls[rc]));
      if (__any(over)) {
        float corr[RC];
#pragma unroll
        for (int rc = 0; rc < RC; ++rc) {
          float mloc = sc[rc][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, sc[rc][i]);
          mloc *= POOLED ? c_pool : c_kept;
          mloc = pair_max(mloc);
          const float m_old = m_run[rc];
          const float m_use = (mloc > m_old + kLazy) ? mloc : m_old;
          corr[rc] = __builtin_amdgcn_exp2f(m_old - m_use);
          m_run[rc] = m_use;
          l_run[rc] *= corr[rc];
        }
#pragma unroll
        for (int rc = 0; rc < RC; ++rc)
#pragma unroll
          for (int dc = 0; dc < 4; ++dc) scale_acc(o[rc][dc], corr[rc]);
        exponentiate(sc, pp, ls);
      }
#pragma unroll
      for (int rc = 0; rc < RC; ++rc) l_run[rc] += ls[rc];
    };

    constexpr int kQkM = (kQk8 ? 2 : 8) * RC;  // MFMAs of one qk(c)
    constexpr int kQkD = kQk8 ? 4 : 8;         // LDS reads of one qk(c)
    constexpr int kPvM = 8 * RC, kPvD = 16;
    f32x16 sa[RC], sb[RC];
    bf16x8 pa[RC][2], pq[RC][2];
    float la[RC], lq[RC];
    // Chunks that are masked for every row of this wave are skipped: in the
    // diagonal tile the keys past the wave's last row, in a pooled tile the
    // pooled keys past block I.  Such tiles run the chunks in plain order.
    int nc = 4;
    if constexpr (DIAG) nc = min(4, tbase / 32 + RC);
    if constexpr (POOLED) nc = min(4, (I - kBlock * tile_index(t)) / 32 + 1);
    if (nc < 4) {
      for (int c = 0; c < nc; ++c) {
        qk(c, sa);
        const bool o1 = softmax(c, sa, pa, la);
        settle(o1, sa, pa, la);
        pv(c, pa);
      }
      publish_slot(t + 2, page_next, buf);
      wait_vm();
      __syncthreads();
      return;
    }
    qk(0, sa);
    __builtin_amdgcn_sched_barrier(0);
    qk(1, sb);
    bool ov = softmax(0, sa, pa, la);
    interleave<kQkM, kQkD>();
    settle(ov, sa, pa, la);
    qk(2, sa);
    pv(0, pa);
    ov = softmax(1, sb, pq, lq);
    interleave<kQkM + kPvM, kQkD + kPvD>();
    settle(ov, sb, pq, lq);
    qk(3, sb);
    pv(1, pq);
    ov = softmax(2, sa, pa, la);
    interleave<kQkM + kPvM, kQkD + kPvD>();
    settle(ov, sa, pa, la);
    pv(2, pa);
    ov = softmax(3, sb, pq, lq);
    interleave<kPvM, kPvD>();
    settle(ov, sb, pq, lq);
    pv(3, pq);

    publish_slot(t + 2, page_next, buf);
    wait_vm();
    __syncthreads();
  };

  // lists are ascending and end with the diagonal block: off-diagonal kept
  // tiles, then the diagonal tile (causal mask), each in a loop of its own
  const bool last_is_diag = nkept > 0 && tile_index(nkept - 1) == I;
  const int n_off = last_is_diag ? nkept - 1 : nkept;
  for (int t = tbeg; t < min(n_off, tend); ++t) iterate(t, std::false_type{}, std::false_type{});
  if (last_is_diag && nkept - 1 >= tbeg && nkept - 1 < tend)
    iterate(nkept - 1, std::false_type{}, std::true_type{});
  if constexpr (kFp8) {
    // pooled tiles run on bf16 MFMA: widen the fp8 Q fragments (exact)
#pragma unroll
    for (int rc = 0; rc < RC; ++rc)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int k2 = kk >> 2, w0 = 2 * (kk & 3);
        const unsigned wlo = (unsigned)qf8[rc][k2][w0], whi = (unsigned)qf8[rc][k2][w0 + 1];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          qf[rc][kk][i] = f32_to_bf16(e4m3_to_f32(((i < 4 ? wlo : whi) >> (8 * (i & 3))) & 0xFFu));
      }
  }
  for (int t = max(nkept, tbeg); t < tend; ++t) iterate(t, std::true_type{}, std::false_type{});

  // The lane's row index again, opaque to the compiler: otherwise it keeps
  // the 64-bit row addresses of the Q loads live through the whole loop
  // (two register pairs, which spill in the e4m3 instances).
  int ecol = col;
  asm volatile("" : "+v"(ecol));
  if (a.splits > 1) {
    // part of a split row: O_part = acc / l and lse_part in fp32 for the
    // combine pass (an empty part: O_part = 0, lse_part = -inf)
#pragma unroll
    for (int rc = 0; rc < RC; ++rc) {
      const float l_tot = l_run[rc] + __shfl_xor(l_run[rc], 32, 64);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (ecol >= nvalid[rc]) continue;
      const int64_t tok = tok0 + tbase + 32 * rc + ecol;
      float* ob = a.opart + (((int64_t)split * a.total_tokens + tok) * a.hq + hq_idx) * kHeadDim;
#pragma unroll
      for (int dc = 0; dc < 4; ++dc)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(ob + 32 * dc + 8 * j + 4 * half) =
              make_float4(o[rc][dc][4 * j] * inv, o[rc][dc][4 * j + 1] * inv,
                          o[rc][dc][4 * j + 2] * inv, o[rc][dc][4 * j + 3] * inv);
      if (half == 0)
        a.lpart[((int64_t)split * a.hq + hq_idx) * a.total_tokens + tok] =
            l_tot > 0.f ? (m_run[rc] + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }

  // ---- epilogue: O = acc / l, lse = m + log2(l) (natural log out) ----
  if constexpr (kFp8) {
    // direct stores (the e4m3 instances keep their register budget for the
    // loops; the staged form below adds pressure that spills there)
#pragma unroll
    for (int rc = 0; rc < RC; ++rc) {
      const float l_tot = l_run[rc] + __shfl_xor(l_run[rc], 32, 64);
      const float inv = 1.f / l_tot;
      if (ecol >= nvalid[rc]) continue;
      const int64_t tok = tok0 + tbase + 32 * rc + ecol;
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
    return;
  }
  // Each wave stages its rows in LDS (the tile buffers are free after the
  // last barrier; every wave owns a region of its own, so no barrier is
  // needed) with 16-byte chunks XOR-swizzled by row, then writes whole output
  // rows: 16 bytes per lane, 4 (bf16) or 2 (fp32) rows per store instruction.
  constexpr int kOutB = (ODT == FP_BF16) ? 2 : 4;                 // bytes per output element
  constexpr int kRowChunks = kHeadDim * kOutB / 16;               // 16-byte chunks per row
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = reinterpret_cast<uint8_t*>(&sm.k[0][0]) + wv * (32 * RC * kHeadDim * kOutB);
#pragma unroll
  for (int rc = 0; rc < RC; ++rc) {
    const float l_tot = l_run[rc] + __shfl_xor(l_run[rc], 32, 64);
    const float inv = 1.f / l_tot;
    const int r = 32 * rc + col;  // row inside the wave's block of rows
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dc + 8 * j + 4 * half;
        const float x0 = o[rc][dc][4 * j] * inv, x1 = o[rc][dc][4 * j + 1] * inv;
        const float x2 = o[rc][dc][4 * j + 2] * inv, x3 = o[rc][dc][4 * j + 3] * inv;
        const int byte = d * kOutB;              // within the row
        const int ch = byte >> 4, in = byte & 15;
        uint8_t* dst = stage + r * (kHeadDim * kOutB) + ((ch ^ (r & (kRowChunks - 1))) << 4) + in;
        if constexpr (ODT == FP_BF16) {
          *reinterpret_cast<uint2*>(dst) = f32x4_to_bf16x4(make_float4(x0, x1, x2, x3));
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(x0, x1, x2, x3);
        }
      }
    }
    if (a.lse && half == 0 && col < nvalid[rc])
      a.lse[(int64_t)hq_idx * a.total_tokens + tok0 + tbase + r] = (m_run[rc] + __log2f(l_tot)) * kLn2;
  }
  // read back whole rows (the wave's own LDS writes are ordered before its reads)
  constexpr int kRowsPerStore = 64 / kRowChunks;
  int nrows_w = 0;  // valid rows of this wave (chunks fill in order)
#pragma unroll
  for (int rc = 0; rc < RC; ++rc) nrows_w += nvalid[rc];
#pragma unroll
  for (int it = 0; it < 32 * RC / kRowsPerStore; ++it) {
    const int r = it * kRowsPerStore + lane / kRowChunks;
    const int ch = lane % kRowChunks;
    if (r < nrows_w) {
      const uint4 v = *reinterpret_cast<const uint4*>(stage + r * (kHeadDim * kOutB) +
                                                      ((ch ^ (r & (kRowChunks - 1))) << 4));
      const int64_t tok = tok0 + tbase + r;
      uint8_t* gdst = reinterpret_cast<uint8_t*>(a.out) + ((tok * a.hq + hq_idx) * (int64_t)kHeadDim) * kOutB + ch * 16;
      *reinterpret_cast<uint4*>(gdst) = v;
    }
  }
}

// KV-split combine ("長文本推理越來越長但你的顯卡等不起…FlashPrefill V2",
// KV-split load-balancing passage): the parts of a row, each normalised by
// its own sum, are merged by their log-sum-exp,
//   lse = ln sum_s e^{lse_s},  O = sum_s e^{lse_s - lse} O_s.
// One wave per (token, query head), two head-dim elements per lane.
template <int ODT>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ opart,
                                                           const float* __restrict__ lpart, int splits,
                                                           int64_t T, int hq, void* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= T * hq) return;
  const int lane = threadIdx.x & 63;
  const int64_t tok = pair / hq;
  const int hh = (int)(pair % hq);
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, lpart[((int64_t)s * hq + hh) * T + tok]);
  float tot = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float w = expf(lpart[((int64_t)s * hq + hh) * T + tok] - m);  // empty part: 0
    const float2 v = *reinterpret_cast<const float2*>(opart + (((int64_t)s * T + tok) * hq + hh) * kHeadDim + 2 * lane);
    tot += w;
    o0 = fmaf(w, v.x, o0);
    o1 = fmaf(w, v.y, o1);
  }
  const float inv = 1.f / tot;
  const int64_t e = (tok * hq + hh) * kHeadDim + 2 * lane;
  if constexpr (ODT == FP_BF16) {
    const bf16x2 b = bf16x2{f32_to_bf16(o0 * inv), f32_to_bf16(o1 * inv)};
    *reinterpret_cast<bf16x2*>(reinterpret_cast<u16*>(out) + e) = b;
  } else {
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + e) = make_float2(o0 * inv, o1 * inv);
  }
  if (lse && lane == 0) lse[(int64_t)hh * T + tok] = m + logf(tot);
}

// Block offsets of the map and the attention's item counter (last block of
// the grid) and bf16 copies of the pooled keys / values (each rounded once
// from float64).
__global__ __launch_bounds__(256) void attn_prep_kernel(SeqMap m, const double* __restrict__ km,
                                                        const double* __restrict__ vm, u16* __restrict__ km16,
                                                        u16* __restrict__ vm16, int64_t n, int* __restrict__ queue) {
  if (blockIdx.x == gridDim.x - 1) {
    if (threadIdx.x == 0) *queue = 0;  // the attention kernel's item counter
    plan_offsets(m);
    return;
  }
  if (km == nullptr) return;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const double2* kp = reinterpret_cast<const double2*>(km + i);
  const double2* vp = reinterpret_cast<const double2*>(vm + i);
  const double2 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
  const ushort4 kb = make_ushort4(f64_to_bf16_bits(k0.x), f64_to_bf16_bits(k0.y),
                                  f64_to_bf16_bits(k1.x), f64_to_bf16_bits(k1.y));
  const ushort4 vb = make_ushort4(f64_to_bf16_bits(v0.x), f64_to_bf16_bits(v0.y),
                                  f64_to_bf16_bits(v1.x), f64_to_bf16_bits(v1.y));
  *reinterpret_cast<ushort4*>(km16 + i) = kb;
  *reinterpret_cast<ushort4*>(vm16 + i) = vb;
}

}  // namespace

hipError_t launch_attn_prep(const Geometry& g, const SeqMap& m, const double* k_mean,
                            const double* v_mean, u16* km16, u16* vm16, int* queue, hipStream_t st) {
  const int64_t n = (int64_t)g.hkv * g.num_blocks * kHeadDim;
  const unsigned conv = k_mean ? (unsigned)((n / 4 + 255) / 256) : 0u;
  hipLaunchKernelGGL(attn_prep_kernel, dim3(conv + 1), dim3(256), 0, st, m, k_mean, v_mean, km16,
                     vm16, n, queue);
  return hipGetLastError();
}

int attn_splits(const Geometry& g) {
  if (g.attn_splits > 0) return std::min(g.attn_splits, kAttnMaxSplits);
  const int64_t wgs = ((g.lists * g.num_qblocks + 7) / 8) * 8 * ((g.lgroup + 1) / 2);
  if (2 * wgs > kAttnSplitTarget) return 1;
  return (int)std::min<int64_t>(kAttnMaxSplits, kAttnSplitTarget / wgs);
}

hipError_t launch_attn(const Geometry& g, const SeqMap& m, const int32_t* page_table, const void* q,
                       const void* k_cache, const void* v_cache, const float* q_scale,
                       const float* k_scale, const int32_t* row_ptr, const int32_t* col_idx,
                       const u16* km16, const u16* vm16, int correction, void* out, float* lse,
                       float* opart, float* lpart, int* queue, hipStream_t st, bool dense) {
  AttnArgs a;
  a.m = m;
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
  a.splits = attn_splits(g);
  a.opart = opart;
  a.lpart = lpart;
  if (a.splits > 1 && (!opart || !lpart)) return hipErrorInvalidValue;
  a.num_blocks = g.num_blocks;
  a.num_qblocks = g.num_qblocks;
  a.total_tokens = g.total_tokens;
  a.max_pages = g.max_pages;
  a.page_size = g.page_size;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.group = g.lgroup;
  a.lists = g.lists;
  a.kvdiv = g.kvdiv;
  a.packs = (g.lgroup + 1) / 2;
  a.correction = dense ? 0 : correction;
  a.softmax_scale = g.softmax_scale;
  const int64_t rows = (int64_t)g.lists * g.num_qblocks;
  const int64_t nitems = ((rows + 7) / 8) * 8 * a.packs * a.splits;
  if (nitems > INT32_MAX / 2) return hipErrorInvalidValue;
  // Launches of many waves per CU hand their last kAttnDynFrac items out on
  // demand, with kAttnDynSlack of that count in extra workgroups; small
  // launches keep the static order.
  int64_t ndyn = 0, slack = 0;
  if (nitems >= kAttnDynMinItems) {
    ndyn = nitems * kAttnDynFracPct / 100;
    slack = ndyn * kAttnDynSlackPct / 100;
  }
  a.nitems = (int)nitems;
  a.dyn_begin = (int)(nitems - ndyn);
  a.queue = queue;
  const unsigned grid = (unsigned)(nitems + slack);
  const size_t shm = sizeof(SharedMem);
#define FP_ATTN_D(QD, VD, OD, DN)                                                              \
  do {                                                                                         \
    static std::atomic<uint64_t> smem_set;                                                     \
    const hipError_t ea =                                                                      \
        set_smem_limit(smem_set, (const void*)attn_kernel<QD, VD, OD, kAttnWaves, DN>, shm);   \
    if (ea != hipSuccess) return ea;                                                           \
    hipLaunchKernelGGL((attn_kernel<QD, VD, OD, kAttnWaves, DN>), dim3(grid), dim3(64 * kAttnWaves), \
                       shm, st, a);                                                            \
  } while (0)
#define FP_ATTN(QD, VD, OD)                    \
  do {                                         \
    if (dense) FP_ATTN_D(QD, VD, OD, true);    \
    else FP_ATTN_D(QD, VD, OD, false);         \
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
#undef FP_ATTN_D
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t pairs = g.total_tokens * g.hq;
  const unsigned cgrid = (unsigned)((pairs + 3) / 4);
  if (g.out_dtype == FP_BF16)
    hipLaunchKernelGGL(attn_combine_kernel<FP_BF16>, dim3(cgrid), dim3(256), 0, st, opart, lpart,
                       a.splits, g.total_tokens, g.hq, out, lse);
  else
    hipLaunchKernelGGL(attn_combine_kernel<FP_F32>, dim3(cgrid), dim3(256), 0, st, opart, lpart,
                       a.splits, g.total_tokens, g.hq, out, lse);
  return hipGetLastError();
}

}  // namespace fp
