// Lightning Indexer scores: I(t, s) = sum_h w[t][h] * max(0, q_I[t][h] . k_I[s])
// for every compressed entry s visible to query t (s < floor(t/m)).
//
// Method: shareware.cn Hybrid Attention article, sections 六-七 (a cheap
// scorer with few heads and a small head dim, per-head ReLU before the head
// sum); trdm.cn attention article, section 4.2 (relu of q_idx against the
// pooled index keys, the key shared by all indexer heads).
//
// Design (gfx950, bf16): in decode the scan over all index keys is the
// dominant HBM stream (256 B per key at d_I = 128) while each key costs
// H_I * d_I MACs, i.e. 64 flop per byte at H_I = 64: above the fp32 VALU
// ridge, so the dot products run on MFMA (v_mfma_f32_16x16x32_bf16, A = the
// query's H_I x d_I indexer block held in VGPRs, B = 16 keys, 16 heads x 16
// keys per block).  Each wavefront streams one contiguous key range through a
// private LDS ring of 16-key tiles filled by direct-to-LDS loads (a 4 KiB
// tile = four 1 KiB wave loads, several tiles in flight); the 16-byte pieces
// of each key are placed XOR-swizzled by the load addresses so that the MFMA
// operand reads hit distinct LDS banks.  In the 16x16 output layout a lane
// holds one key column and 4 head rows per block, so the ReLU and the
// weighted head sum are in-register FMAs plus two lane exchanges; the
// epilogue writes 16 fp32 scores (64 B) per tile.  The grid is about one
// workgroup per CU, so every wavefront streams megabytes with one prologue.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"
#include "merge.hpp"
#include "select.hpp"

namespace csa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
#ifndef CSA_INDEX_DEPTH
#define CSA_INDEX_DEPTH 6
#endif
constexpr int kTileKeys = 16;                 // keys per MFMA tile (the N dimension)
constexpr int kDepth = CSA_INDEX_DEPTH;       // ring slots per wavefront (kDepth - 1 tiles in flight)
constexpr int kTileBytes = kTileKeys * 256;   // d_I = 128 bf16 keys
// FP8 keys (128 B): tiles of half the size.
constexpr int kTileBytes8 = kTileKeys * 128;
// MXFP4 keys (64 code bytes + 4 E8M0 scales): a tile is its 1 KiB of codes
// and four copies of its 64 scale bytes (one dword load).
constexpr int kTileBytes4 = kTileKeys * 64 + 256;
// FP8 and MXFP4 scans run two wavefronts per SIMD (8 per workgroup), so that
// one wavefront's per-tile chain (LDS read, MFMA, ReLU / weight / head-sum
// epilogue) overlaps another's; each keeps half the ring slots (the same
// bytes in flight per CU).  A workgroup still scans 4 * per_wave keys.
constexpr int kWaves8 = 8;
constexpr int kDepthW8 = kDepth;  // FP8 slots per wavefront with 8 wavefronts
constexpr int kDepthW4 = 8;       // MXFP4
static_assert(kWaves8 * kDepthW8 * kTileBytes8 == kWaves * kDepth * kTileBytes, "FP8 ring of the bf16 size");
static_assert(kWaves8 * kDepthW4 * kTileBytes4 <= kWaves * kDepth * kTileBytes, "MXFP4 ring fits the same space");
constexpr int kMinKeysPerWave = 256;
constexpr int kMaxKeysPerWave = 3968;         // scores of a workgroup stay in LDS (62 KiB)
constexpr int kMaxTiles = kMaxKeysPerWave / kTileKeys;
constexpr int kDirectTiles = 16;  // tiles per wavefront of the d_I = 64 kernel
constexpr int kDirectKeysPerWg = kWaves * kDirectTiles * kTileKeys;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most LPT * n of this wave's loads are outstanding (LPT loads
// per tile, n < ring depth).
// max(0, x) as one signed-integer max on the bits: a float with the sign bit
// set is a negative integer and becomes +0; others are unchanged (fmaxf would
// first canonicalise its input, one more instruction per value).  Equal to
// fmaxf(x, 0) for every non-NaN x.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// A key's score from a wavefront's 16 x 16 MFMA blocks (heads as rows):
// lane (g, c16) holds heads 16 mb + 4g + r of key c16.  head_part sums w_h *
// ReLU(q_h . k) over the lane's 4 MB heads as two FMA chains (r = 0, 1 and
// r = 2, 3), one VALU instruction per head after the ReLU; group_sum4_pair
// then adds the four lane groups.  The decode scan and the 16-row prefill
// scorer both use them, so a query's scores are the same bit for bit
// whichever kernel computes them.
template <int MB, bool HAS_W>
__device__ __forceinline__ float head_part(const f32x4 (&acc)[MB], const float (&wr)[MB][HAS_W ? 4 : 1]) {
  float sa, sb;
  if constexpr (HAS_W) {
    sa = __builtin_fmaf(wr[0][1], relu_bits(acc[0][1]), wr[0][0] * relu_bits(acc[0][0]));
    sb = __builtin_fmaf(wr[0][3], relu_bits(acc[0][3]), wr[0][2] * relu_bits(acc[0][2]));
#pragma unroll
    for (int mb = 1; mb < MB; ++mb) {
      sa = __builtin_fmaf(wr[mb][0], relu_bits(acc[mb][0]), sa);
      sb = __builtin_fmaf(wr[mb][2], relu_bits(acc[mb][2]), sb);
      sa = __builtin_fmaf(wr[mb][1], relu_bits(acc[mb][1]), sa);
      sb = __builtin_fmaf(wr[mb][3], relu_bits(acc[mb][3]), sb);
    }
  } else {
    sa = relu_bits(acc[0][0]) + relu_bits(acc[0][1]);
    sb = relu_bits(acc[0][2]) + relu_bits(acc[0][3]);
#pragma unroll
    for (int mb = 1; mb < MB; ++mb) {
      sa = (sa + relu_bits(acc[mb][0])) + relu_bits(acc[mb][1]);
      sb = (sb + relu_bits(acc[mb][2])) + relu_bits(acc[mb][3]);
    }
  }
  return sa + sb;
}

// Sums over the four 16-lane groups of two values at once, each as
// (g0 + g2) + (g1 + g3): the upper half-wave's values meet the lower half's
// (x0's in lanes 0-31, x1's in lanes 32-63), then odd rows meet even rows.
// Lanes of groups 0 and 1 end with x0's total, groups 2 and 3 with x1's; with
// x1 = x0 every lane holds x0's total, the same bits (additions commute).
__device__ __forceinline__ float group_sum4_pair(float x0, float x1) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const uint32_t v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int LPT>
__device__ __forceinline__ void wait_tiles(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<LPT * 1>(); break;
    case 2: wait_vmcnt<LPT * 2>(); break;
    case 3: wait_vmcnt<LPT * 3>(); break;
    case 4: wait_vmcnt<LPT * 4>(); break;
    case 5: wait_vmcnt<LPT * 5>(); break;
    case 6: wait_vmcnt<LPT * 6>(); break;
    case 7: wait_vmcnt<LPT * 7>(); break;
    case 8: wait_vmcnt<LPT * 8>(); break;
    case 9: wait_vmcnt<LPT * 9>(); break;
    case 10: wait_vmcnt<LPT * 10>(); break;
    case 11: wait_vmcnt<LPT * 11>(); break;
    case 12: wait_vmcnt<LPT * 12>(); break;
    case 13: wait_vmcnt<LPT * 13>(); break;
    default: wait_vmcnt<LPT * 14>(); break;
  }
  asm volatile("" ::: "memory");
}
static_assert(kDepth >= 2 && kDepth <= 15 && kDepthW4 <= 15, "wait_tiles covers up to 14 tiles in flight");
static_assert(4 * (kDepth - 1) < 64 && 2 * (kDepthW8 - 1) < 64 && 2 * (kDepthW4 - 1) < 64, "vmcnt range");

// 16 bytes per lane, global -> LDS at lds + 16 * lane (lds wave-uniform, via
// M0), nontemporal (every key is read once: streaming through the caches
// with nt measured 7.1 TB/s against 5.8 TB/s without on a 1 GiB scan).
// Inline asm on purpose: the compiler then adds no implicit "drain all
// loads" before later LDS reads; completion is awaited with explicit vmcnt
// waits.  The instruction writes no registers; M0 is restored.  The first
// form takes a wave-uniform base and a 32-bit lane offset, the second a full
// per-lane address.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* lds) {
  typedef const uint8_t __attribute__((address_space(3))) * lds_ptr;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
}
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, const uint8_t* lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sbase), "s"(lds_addr(lds))
               : "memory");
}
__device__ __forceinline__ void dma16(const void* g, const uint8_t* lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(lds_addr(lds))
               : "memory");
}
// The same with 4 bytes per lane (lane i's dword lands at lds + 4i).
__device__ __forceinline__ void dma4(const char* sbase, uint32_t voff, const uint8_t* lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dword %1, %2 nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sbase), "s"(lds_addr(lds))
               : "memory");
}
__device__ __forceinline__ void dma4(const void* g, const uint8_t* lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(lds_addr(lds))
               : "memory");
}

// Sum of x over the four 16-lane groups (lanes c, c+16, c+32, c+48), in every
// lane, by the gfx950 row-swap permutes (no LDS round trip).
// Fused top-k, part stage: the workgroup's part of the row (nkv visible keys
// starting at key kb, scores in LDS in the tile layout of the scan) keeps its
// top-min(cap, nkv) entries, written as index-ordered (score, index) pairs in
// candidate slot `slot`, with their count.  Any entry of the row's top-k is
// in its part's top-k (fewer entries beat it inside the part than in the whole
// row), ties included.  The tile ring is free at this point and holds the
// selection's state.
template <int NW>
using PartSel = sel::Filter<64 * NW, 64 * kWaves / NW, NW == kWaves ? 24 : 16>;
constexpr int kPartKeys = 64 * kWaves * 64;  // 16384 >= 4 * kMaxKeysPerWave
constexpr int kCandStage = 2048;             // largest cap staged in LDS
constexpr int kListStage = 1024;             // largest compact list staged in LDS
static_assert(4 * kMaxKeysPerWave <= kPartKeys, "a part fits the selection tile");
static_assert(kListStage >= kListMax, "the longest list fits its LDS stage");
static_assert(sizeof(PartSel<kWaves>::Shared) + (kCandStage + 64) * 8 + (kListStage + 64) * 8 <=
                  kWaves * kDepth * kTileBytes,
              "selection state fits the ring");
static_assert(sizeof(PartSel<kWaves8>::Shared) + (kCandStage + 64) * 8 + (kListStage + 64) * 8 <=
                  kWaves8 * kDepthW4 * kTileBytes4,
              "selection state fits the 8-wavefront rings");
// Score slots per wavefront: a workgroup's range holds at most
// 4 * kMaxKeysPerWave keys, split over NW wavefronts.
template <int NW>
constexpr int kScoreSlots = kMaxTiles * kWaves / NW * kTileKeys;

// Position of key c (0..15) of a wavefront's tile `it` in its score list: the
// four 4-key chunks of a tile are rotated by the tile number, so that 16 lanes
// reading chunk q of 16 consecutive tiles (one 16-byte read each) hit 16
// different bank groups.
__device__ __forceinline__ int sb_pos(int it, int c) { return it * kTileKeys + ((((c >> 2) + it) & 3) << 2) + (c & 3); }

// Score of key o of the workgroup's range: tile T = o / 16 is tile T / NW of
// wavefront T % NW.
template <int NW>
__device__ __forceinline__ float part_score(const float (*sbuf)[kScoreSlots<NW>], int o) {
  const int T = o / kTileKeys;
  return sbuf[T % NW][sb_pos(T / NW, o % kTileKeys)];
}

// Compact lists: a row with P non-empty parts (nv visible entries, part_keys
// keys per part) lists ceil(2k / P) per part; with P * cap <= kMergeUnion its
// parts hand the merge their whole candidate sets (count kWholePart).
template <int NW>
__device__ __forceinline__ void part_select(const IndexCandidates& co, int64_t slot, int64_t kb, int nkv,
                                            int64_t nv, int64_t part_keys,
                                            const float (*sbuf)[kScoreSlots<NW>], uint8_t* scratch) {
  using PS = PartSel<NW>;
  constexpr int IT = kPartKeys / (64 * NW);  // entries per thread
  constexpr int TPT = IT / kTileKeys;        // tiles per thread
  constexpr int MT = kScoreSlots<NW> / kTileKeys;
  const int tid = threadIdx.x;
  const int cap = static_cast<int>(co.cap);
  float* ov = co.cval + slot * co.cap;
  int32_t* oi = co.cidx + slot * co.cap;
  if (nkv <= cap) {  // the whole part is kept; the rest of the slots hold NaN (no candidate)
    for (int o = tid; o < cap; o += 64 * NW) {
      ov[o] = o < nkv ? part_score<NW>(sbuf, o) : __builtin_nanf("");
      if (o < nkv) oi[o] = static_cast<int32_t>(kb + o);
    }
    if (tid == 0) {
      co.ccnt[slot] = nkv;
      if (co.lval) {  // no compact list: an empty part contributes nothing, a short one its whole candidate set
        co.lcnt[slot] = nkv == 0 ? 0 : mrg::kWholePart;
        co.lthr[slot] = -INFINITY;
      }
    }
    return;
  }
  typename PS::Shared& ss = *reinterpret_cast<typename PS::Shared*>(scratch);
  int32_t* si = reinterpret_cast<int32_t*>(scratch + sizeof(typename PS::Shared));
  float* sv = reinterpret_cast<float*>(si + kCandStage + 64);  // each array: 64 dump slots at its end
  int32_t* li = reinterpret_cast<int32_t*>(sv + kCandStage + 64);
  float* lv = reinterpret_cast<float*>(li + kListStage + 64);
  const uint32_t lane = threadIdx.x & 63;
  const int lcap = static_cast<int>(co.lcap);  // <= kListStage
  const int64_t prow = nv > 0 ? (nv + part_keys - 1) / part_keys : 1;  // the row's non-empty parts
  const bool whole = co.lval && prow * co.cap <= kMergeUnion;
  int64_t rrow = (2 * co.cap + prow - 1) / prow;
  if (rrow > co.cap) rrow = co.cap;
  PS::zero(ss);
  // Thread t holds entries IT*t .. IT*t+IT-1 of the part: tiles TPT*t ..
  // TPT*t+TPT-1 (tile T is tile T / NW of wavefront T % NW), 16 consecutive
  // scores each; entries past the visible ones are NaN (never selected).
  float x[IT];
  const int o0 = tid * IT;
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int T = TPT * tid + j;
    const int w = T % NW;
    const int tl = T / NW < MT ? T / NW : MT - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(&sbuf[w][sb_pos(tl, 4 * q)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[j * 16 + 4 * q + e] = v[e];
    }
  }
#pragma unroll
  for (int j = 0; j < IT; ++j) x[j] = o0 + j < nkv ? x[j] : __builtin_nanf("");
  float vmin, vmax;
  PS::block_range(x, ss, &vmin, &vmax);
  float thr2 = -INFINITY;
  uint32_t cnt2 = 0;
  PS::run2(
      x, [&](uint32_t e) { return part_score<NW>(sbuf, static_cast<int>(e) < nkv ? static_cast<int>(e) : 0); },
      static_cast<uint32_t>(nkv), static_cast<uint32_t>(cap), vmin, vmax, ss,
      [&](uint32_t pos, float v, uint32_t e) {
        const uint32_t p = pos != sel::kNoSlot ? pos : kCandStage + lane;  // lane-private dump slot
        si[p] = static_cast<int32_t>(e);
        sv[p] = v;
      },
      [&](int j, uint32_t pos) {
        si[pos] = o0 + j;
        sv[pos] = part_score<NW>(sbuf, o0 + j);
      },
      co.lval && !whole ? static_cast<uint32_t>(rrow) : 0u,
      [&](uint32_t pos, float v, uint32_t e) {
        const uint32_t p = pos < static_cast<uint32_t>(lcap) ? pos : kListStage + lane;  // past lcap: dropped
        li[p] = static_cast<int32_t>(e);
        lv[p] = v;
      },
      &thr2, &cnt2);
  for (int i = tid; i < cap; i += 64 * NW) {
    ov[i] = sv[i];
    oi[i] = static_cast<int32_t>(kb + si[i]);
  }
  if (co.lval && whole) {
    if (tid == 0) {
      co.lcnt[slot] = mrg::kWholePart;
      co.lthr[slot] = -INFINITY;
    }
  } else if (co.lval) {
    const bool fits = cnt2 <= static_cast<uint32_t>(lcap);
    if (fits) {
      for (int i = tid; i < static_cast<int>(cnt2); i += 64 * NW) {
        co.lval[slot * co.lcap + i] = lv[i];
        co.lidx[slot * co.lcap + i] = static_cast<int32_t>(kb + li[i]);
      }
    }
    if (tid == 0) {
      co.lcnt[slot] = fits ? static_cast<int32_t>(cnt2) : -1;
      co.lthr[slot] = thr2;
    }
  }
  if (tid == 0) co.ccnt[slot] = cap;
}

// Exact short list of a part of at most kListPartKeys keys, for the listed
// path: every visible entry whose score is >= V, V the part's r-th largest
// score (r = co.lrank; every entry when the part holds at most r, V = -inf),
// in index order, with its count and V.  More than co.lcap entries (ties at
// V) leave no list (count -1).  V comes from a radix select on
// order-preserving keys, four 8-bit digits (one wavefront reads 4 bins per
// lane with one 16-byte LDS read); the bins and the per-pass results live in
// the idle tile ring.
// Two size classes: ranges of up to 1,024 keys (batch 1 at 1M, batch 8 at
// 131,072) and up to 4,096 (batch 2 and 4 at 1M).
constexpr int kListPartKeys = 1024;
constexpr int kListPartKeysMax = 4096;
template <int NW, int KEYS>
__device__ __forceinline__ void part_list(const IndexCandidates& co, int64_t slot, int64_t kb, int n,
                                          const float (*sbuf)[kScoreSlots<NW>], uint8_t* scratch) {
  constexpr int NT = 64 * NW;
  constexpr int IT = KEYS / NT;  // entries per thread (4 or 16 with four wavefronts, half with eight)
  static_assert(IT >= 1 && IT <= 32 && KEYS % NT == 0, "entries per thread fit the 32-bit masks");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t r = static_cast<uint32_t>(co.lrank);
  uint32_t* hist = reinterpret_cast<uint32_t*>(scratch);  // two sets of 256 bins
  uint32_t* pick = hist + 512;                             // per set: digit, entries above it, entries in it
  uint32_t* wsum = pick + 8;                               // per-wavefront counts
  float x[IT];
  uint32_t key[IT];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int o = tid * IT + j;
    x[j] = part_score<NW>(sbuf, o < n ? o : 0);
    key[j] = float_key(x[j]);
    valid |= static_cast<uint32_t>(o < n) << j;
  }
  const bool keep_all = static_cast<uint32_t>(n) <= r;
  uint32_t kth = 0;  // every valid key >= kth is listed
  if (!keep_all) {
    // four 8-bit digits, most significant first; bins double-buffered so
    // that one pass's counting can follow the previous pass's search.  When
    // the chosen bin holds exactly the entries still needed, every key at or
    // above the bin's lowest key is listed and the search stops there (V is
    // then that lower bound, at most the r-th largest score).
    uint32_t prefix = 0, mask = 0, need = r;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint32_t* h = hist + 256 * (pass & 1);
#pragma unroll
      for (int j = 0; j < IT; ++j)
        if (((valid >> j) & 1) && (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> shift) & 255u], 1u);
      hist[256 * ((pass + 1) & 1) + (tid & 255)] = 0;  // the next pass's bins
      __syncthreads();
      if (wave == 0) {  // lane l holds bins 255-4l .. 252-4l (highest first)
        const u32x4 c = *reinterpret_cast<const u32x4*>(h + 252 - 4 * lane);
        const uint32_t sum = c[0] + c[1] + c[2] + c[3];
        uint32_t above = sel::wave_incl_scan(sum) - sum;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (above < need && above + c[q] >= need) {
            pick[4 * (pass & 1)] = static_cast<uint32_t>(252 - 4 * lane + q);
            pick[4 * (pass & 1) + 1] = above;
            pick[4 * (pass & 1) + 2] = c[q];
          }
          above += c[q];
        }
      }
      __syncthreads();
      prefix |= pick[4 * (pass & 1)] << shift;
      mask |= 255u << shift;
      need -= pick[4 * (pass & 1) + 1];
      if (pick[4 * (pass & 1) + 2] == need) break;  // uniform: every entry of the bin is listed
    }
    kth = prefix;
  }
  // ordered compaction of the entries with key >= kth
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < IT; ++j) keep |= static_cast<uint32_t>(((valid >> j) & 1) && (keep_all || key[j] >= kth)) << j;
  const uint32_t cnt = static_cast<uint32_t>(__builtin_popcount(keep));
  const uint32_t incl = sel::wave_incl_scan(cnt);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t pos = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    pos += w < wave ? wsum[w] : 0u;
    total += wsum[w];
  }
  const bool fits = total <= static_cast<uint32_t>(co.lcap);
  if (fits) {
    float* lv = co.lval + slot * co.lcap;
    int32_t* li = co.lidx + slot * co.lcap;
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      if ((keep >> j) & 1) {
        lv[pos] = x[j];
        li[pos] = static_cast<int32_t>(kb + tid * IT + j);
        ++pos;
      }
    }
  }
  if (tid == 0) {
    co.lcnt[slot] = fits ? static_cast<int32_t>(total) : -1;
    co.lthr[slot] = keep_all ? -INFINITY : key_float(kth);
  }
}

// d_I = 128 (KS = 4), MB = H_I / 16 head blocks.  Workgroup (row, part)
// scores keys [part * 4 * per_wave, +4 * per_wave); with NW wavefronts (4 for
// bf16 keys, 8 for FP8 / MXFP4) wavefront w takes tiles w, w+NW, w+2NW, ...
// so that they stream through adjacent memory.
// Scores collect in LDS and leave in one coalesced pass at the end, so the
// loop issues no stores (their completions would share the load counter the
// ring waits on).
// FP8: keys and queries in OCP E4M3 (128 B per key).  A tile is two 1 KiB
// loads, and one v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit
// scales) per 16-head block takes all 128 dims: lane (g, c) supplies 32
// bytes of row c of each operand, the same bytes for the query and the key,
// so the product is the full dot product (checked on the device against an
// fp64 product of the decoded values, output in the usual 16x16 layout).
// MXFP4: q^I and k^I as E2M1 codes (two per byte, element 2i in the low
// nibble) with one E8M0 scale per 32 elements; the same instruction in its
// FP4 form takes 16 code bytes per lane, and each lane's scale operand is the
// scale of exactly its 32 elements (lane (g, c): row c, block g).
template <int MB, bool HAS_W, bool TOPK, int KF>  // KF: key format, 0 bf16, 1 FP8, 2 MXFP4
__global__ __launch_bounds__(64 * (KF ? kWaves8 : kWaves), 1) void index_score_stream(IndexScoreArgs a, int64_t parts,
                                                                                      int64_t per_wave,
                                                                                      IndexCandidates co) {
  constexpr bool FP8 = KF == 1, FP4 = KF == 2;
  constexpr int NW = KF ? kWaves8 : kWaves;  // wavefronts per workgroup
  constexpr int HI = 16 * MB;
  constexpr int DI = 128;
  constexpr int KS = 4;
  constexpr int KB = FP4 ? 64 : (FP8 ? 128 : 256);                          // code bytes per key
  constexpr int TB = FP4 ? kTileBytes4 : (FP8 ? kTileBytes8 : kTileBytes);  // LDS bytes per tile
  constexpr int DEPTH = FP4 ? kDepthW4 : (FP8 ? kDepthW8 : kDepth);         // ring slots per wavefront
  constexpr int LPT = FP4 ? 2 : TB / 1024;                                  // wave loads per tile
  __shared__ __attribute__((aligned(16))) uint8_t ring[NW][DEPTH][TB];
  __shared__ __attribute__((aligned(16))) float sbuf[NW][kScoreSlots<NW>];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // 16-lane group: k-slots 8g .. 8g+7 of every k-step
  const int c16 = lane & 15;  // key column within the tile
  const int64_t lrow = blockIdx.x / parts;
  const int64_t part = blockIdx.x % parts;
  const int64_t row = a.row0 + lrow;
  const int64_t b = row / a.T;
  const int64_t tpos = seq_len(a.lay, a.n_ctx, a.T, b) - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  float* srow = a.score + lrow * a.ld;

  const int64_t kb = part * kWaves * per_wave;  // first key of the workgroup
  const int64_t ke = kb + kWaves * per_wave < a.L ? kb + kWaves * per_wave : a.L;
  const int64_t kv = ke < nv ? ke : nv;  // keys [kb, kv) are visible
  const int ntiles = kv > kb ? static_cast<int>((kv - kb + kTileKeys - 1) / kTileKeys) : 0;
  const int ntv = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
  const int64_t k0 = kb + static_cast<int64_t>(wave) * kTileKeys;  // first key of this wave's tile 0
  constexpr int64_t kStride = NW * kTileKeys;                        // keys between its tiles

  // Tile layout in LDS.
  //  bf16: key kk (0..15) at kk*256; its 16-byte piece p at slot p ^ kk.
  //    Load j covers keys 4j .. 4j+3 (1 KiB contiguous in HBM); lane l writes
  //    slot l%16 of key 4j + l/16, so it fetches piece (l%16) ^ kk.
  //  FP8: key kk at kk*128, eight 16-byte pieces; lane group g of the MFMA
  //    takes dims 32g .. 32g+31 (pieces 2g and 2g+1).  Piece p of key kk sits
  //    at slot (p + kk/2) % 8, so the 16 keys of one 16-byte read (8 even
  //    keys on one half of the 256-byte bank row, 8 odd keys on the other)
  //    hit 16 distinct bank groups.  Load j covers keys 8j .. 8j+7; lane l
  //    writes slot s = l%8 of key 8j + l/8, so it fetches piece
  //    (s - kk/2) % 8.
  // Only a tile that runs past the last key (the very end of a row) takes
  // per-lane clamped addresses.  A tile's 16 keys are consecutive rows of the
  // key cache: of sequence b's [L] rows, or of one page of a paged pool
  // (pages hold a multiple of 16 entries and tiles start at multiples of 16).
  const char* kpool = static_cast<const char*>(a.k);
  //  MXFP4: key kk's codes at kk*64, four 16-byte blocks; block p of key kk
  //    sits at slot (p + kk/4) % 4 (the 16 keys of one read then cover the 64
  //    banks once).  Lane l of the code load writes slot l%4 of key l/4.
  //    Scales: lane l of the dword load brings key l%16's four scales to
  //    1024 + 4l, i.e. copy l/16; lane group g reads copy g.
  uint32_t voff[LPT];
  int kkl[LPT];  // key of the tile this lane's piece of load j belongs to
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    if constexpr (FP4) {
      const int kk = j == 0 ? lane >> 2 : lane & 15;
      kkl[j] = kk;
      voff[j] = j == 0 ? kk * 64 + ((((lane & 3) - (kk >> 2)) & 3) << 4) : kk * 4;
    } else if constexpr (FP8) {
      const int kk = 8 * j + (lane >> 3), sl = lane & 7;
      kkl[j] = kk;
      voff[j] = kk * 128 + (((sl - (kk >> 1)) & 7) << 4);
    } else {
      kkl[j] = 4 * j + g;
      voff[j] = (4 * j + g) * 256 + ((c16 ^ (4 * j + g)) << 4);
    }
  }
  uint8_t* myring = &ring[wave][0][0];
  // MXFP4 scales follow all code bytes (of B*L keys, or of the pool's
  // npages*page keys), 4 per key.
  const int64_t nkeys = a.lay.bt ? a.lay.npages * a.lay.page : a.B * a.L;
  const char* sbase = FP4 ? kpool + nkeys * KB : nullptr;
  // Paged keys: tiles are issued in order, kStride keys apart, so the page
  // index and the offset of the next tile's first key are walked forward
  // (no division per tile), and each page id is a scalar load (constant
  // address space) made one tile ahead: a vector load of the table would
  // need a vmcnt wait, which would drain the ring, and the scalar load's own
  // wait falls on the loop's LDS wait.  The table is written before the
  // launch; reads stay inside the sequence's table row.
  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  const ConstI32 btrow = a.lay.bt ? (ConstI32)(a.lay.bt + b * a.lay.bt_ld) : nullptr;
  const int64_t bt_last = a.lay.bt ? a.lay.bt_ld - 1 : 0;
  int64_t pw_idx = a.lay.bt ? k0 / a.lay.page : 0;
  int64_t pw_off = a.lay.bt ? k0 - pw_idx * a.lay.page : 0;
  int32_t pw_pg = a.lay.bt ? btrow[pw_idx < bt_last ? pw_idx : bt_last] : 0;
  auto tile_row = [&](int64_t t0) -> int64_t {  // row of key t0; keys t0 .. t0+15 follow it
    if (!a.lay.bt) return b * a.L + t0;
    const int64_t pg = pw_pg < 0 ? 0 : (pw_pg >= a.lay.npages ? a.lay.npages - 1 : pw_pg);
    const int64_t r = pg * a.lay.page + pw_off;
    pw_off += kStride;
    while (pw_off >= a.lay.page) {
      pw_off -= a.lay.page;
      ++pw_idx;
    }
    pw_pg = btrow[pw_idx < bt_last ? pw_idx : bt_last];
    return r;
  };
  auto issue = [&](int it) {
    uint8_t* slot = myring + (it % DEPTH) * TB;
    const int64_t t0 = k0 + static_cast<int64_t>(it) * kStride;
    const int64_t r0 = tile_row(t0);
    if constexpr (FP4) {
      if (t0 + kTileKeys <= a.L) {
        dma16(kpool + r0 * KB, voff[0], slot);
        dma4(sbase + r0 * 4, voff[1], slot + 1024);
      } else {
        int64_t s0 = t0 + kkl[0], s1 = t0 + kkl[1];
        s0 = s0 < a.L - 1 ? s0 : a.L - 1;
        s1 = s1 < a.L - 1 ? s1 : a.L - 1;
        dma16(kpool + (r0 + s0 - t0) * KB + (voff[0] - kkl[0] * KB), slot);
        dma4(sbase + (r0 + s1 - t0) * 4, slot + 1024);
      }
      return;
    }
    if (t0 + kTileKeys <= a.L) {
      const char* tb = kpool + r0 * KB;
#pragma unroll
      for (int j = 0; j < LPT; ++j) dma16(tb, voff[j], slot + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        int64_t s = t0 + kkl[j];
        s = s < a.L - 1 ? s : a.L - 1;
        dma16(kpool + (r0 + s - t0) * KB + (voff[j] - kkl[j] * KB), slot + j * 1024);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < DEPTH - 1; ++i)
    if (i < ntv) issue(i);

  // A operand: query heads (rows) x index dims, resident for the whole kernel.
  bf16x8 afrag[MB][KF ? 1 : KS];
  i32x8 afrag8[MB];
  int qsc[MB];  // MXFP4: E8M0 scale of this lane's 32 query elements
  if constexpr (FP4) {
    const uint8_t* qb = static_cast<const uint8_t*>(a.q);
    const uint8_t* qs = qb + a.B * a.T * HI * 64;  // scales follow all code bytes
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qb + (row * HI + mb * 16 + c16) * 64 + 16 * g);
      afrag8[mb] = i32x8{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]), static_cast<int>(x[3]),
                         0, 0, 0, 0};
      qsc[mb] = qs[(row * HI + mb * 16 + c16) * 4 + g];
    }
  } else if constexpr (FP8) {
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + row * HI * DI;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) afrag8[mb] = *reinterpret_cast<const i32x8*>(qrow + (mb * 16 + c16) * DI + 32 * g);
  } else {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + row * HI * DI;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        afrag[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (mb * 16 + c16) * DI + ks * 32 + g * 8);
  }
  // Head weights for the 4 head rows this lane holds in each 16x16 block.
  float wr[MB][HAS_W ? 4 : 1];
  if (HAS_W) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < (HAS_W ? 4 : 1); ++r) wr[mb][r] = a.w[row * HI + mb * 16 + 4 * g + r];
  }
  // Everything above is in registers / LDS before the loop (so the compiler
  // places no waits inside it); the first tiles have landed too.
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");

  float* sb = sbuf[wave];
  // lane holds S[head mb*16 + 4g + r][key c16] of a tile: ReLU, head
  // weights, and the sum over heads (a short tree in-lane, then across the
  // four lane groups), stored at the tile's score slots.
  // key k0 + it * kStride + c16 is visible iff it * kStride < vlim
  const int64_t vl = nv - k0 - c16;
  const int vlim = vl < 0 ? 0 : (vl > INT32_MAX ? INT32_MAX : static_cast<int>(vl));
  auto finish = [&](int itx, const f32x4 (&acc)[MB]) {
    const float hp = head_part<MB, HAS_W>(acc, wr);
    const float tot = group_sum4_pair(hp, hp);
    if (g == 0) sb[sb_pos(itx, c16)] = itx * static_cast<int>(kStride) < vlim ? tot : -INFINITY;
  };
  for (int it = 0; it < ntv; ++it) {
    if (it + DEPTH - 1 < ntv) {
      issue(it + DEPTH - 1);
      wait_tiles<LPT>(DEPTH - 1);
    } else {
      wait_tiles<LPT>(ntv - 1 - it);
    }
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FP4) {
      const uint8_t* t = myring + (it % DEPTH) * TB;
      const u32x4 x = *reinterpret_cast<const u32x4*>(t + c16 * 64 + (((g + (c16 >> 2)) & 3) << 4));
      const int ksc = static_cast<int>((*reinterpret_cast<const uint32_t*>(t + 1024 + 64 * g + 4 * c16) >> (8 * g)) & 0xffu);
      const i32x8 cur4{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]), static_cast<int>(x[3]), 0, 0, 0, 0};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)  // format 4 = E2M1 for both operands, per-lane E8M0 scales
        acc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag8[mb], cur4, acc[mb], 4, 4, 0, qsc[mb], 0, ksc);
    } else if constexpr (FP8) {
      // Key c16's 128 bytes sit as eight rotated 16-byte blocks; lane (g, c16)
      // takes blocks 2g and 2g+1, i.e. k = 32g .. 32g+31, matching afrag8.
      const uint8_t* t = myring + (it % DEPTH) * TB + c16 * 128;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(t + (((2 * g + (c16 >> 1)) & 7) << 4));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(t + (((2 * g + 1 + (c16 >> 1)) & 7) << 4));
      const i32x8 cur8{static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]), static_cast<int>(x0[3]),
                       static_cast<int>(x1[0]), static_cast<int>(x1[1]), static_cast<int>(x1[2]), static_cast<int>(x1[3])};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)  // format 0 = E4M3 for both operands, scale exponents 127 = 1.0
        acc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag8[mb], cur8, acc[mb], 0, 0, 0, 127, 0, 127);
    } else {
      const uint8_t* t = myring + (it % DEPTH) * TB + c16 * 256;
      bf16x8 cur[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) cur[ks] = *reinterpret_cast<const bf16x8*>(t + (((4 * ks + g) ^ c16) << 4));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[mb][ks], cur[ks], acc[mb], 0, 0, 0);
    }
    finish(it, acc);
  }

  __syncthreads();
  if constexpr (TOPK) {
    part_select<NW>(co, lrow * parts + part, kb, ntiles > 0 ? static_cast<int>(kv - kb) : 0, nv,
                    kWaves * per_wave, sbuf, &ring[0][0][0]);
    return;
  }
  // Write the workgroup's scores [kb, ke) in key order; keys past the visible
  // ones (none in decode) are -inf.  Tile T of the range is tile T/4 of wave
  // T%4; four consecutive keys share a tile, so they move as one 16-byte
  // piece (one LDS read, one store when the row is 16-byte aligned).
  const int nk = static_cast<int>(ke - kb);
  float* dst = srow + kb;
  const bool aligned = (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  for (int o = 4 * static_cast<int>(threadIdx.x); o < nk; o += 4 * 64 * NW) {
    const int T = o / kTileKeys;
    f32x4 x = *reinterpret_cast<const f32x4*>(&sbuf[T % NW][sb_pos(T / NW, o % kTileKeys)]);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (o + e) / kTileKeys < ntiles ? x[e] : -INFINITY;
    if (aligned && o + 4 <= nk) {
      *reinterpret_cast<f32x4*>(dst + o) = x;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (o + e < nk) dst[o + e] = x[e];
    }
  }
  // listed path (ranges of at most kListPartKeysMax keys): the range's exact list
  if (co.lval != nullptr) {
    const int nvis = ntiles > 0 ? static_cast<int>(kv - kb) : 0;
    if (nk <= kListPartKeys)
      part_list<NW, kListPartKeys>(co, lrow * parts + part, kb, nvis, sbuf, &ring[0][0][0]);
    else
      part_list<NW, kListPartKeysMax>(co, lrow * parts + part, kb, nvis, sbuf, &ring[0][0][0]);
  }
}

// Prefill scoring (bf16, FP8 or MXFP4, d_I = 128): a workgroup takes 16 query
// rows of one sequence, two per wavefront with their query blocks resident as
// MFMA A operands, and a part of up to kMultiKeys keys.  Each 16-key tile is
// staged once in LDS (bf16: waves 0-3 load 1 KiB each; FP8: waves 0-1;
// MXFP4: wave 0 loads the codes and the scales; a ring of up to 32 KiB, one
// barrier per two tiles) and read by all 8 wavefronts, each
// B fragment feeding both rows' MFMAs, so a key leaves the caches once per 16
// queries.  Tile layout, MFMA order and epilogue are the streaming scan's, so
// the scores are bit-identical.  Scores collect in LDS and leave at the end
// (no stores in the loop); keys past a row's visible ones get -inf.
constexpr int kMultiRows = 16;
constexpr int kMultiRpw = 2;  // rows per wavefront
constexpr int kMultiDepth = 8;  // bf16 ring slots (FP8: twice as many half-size tiles)
constexpr int kMultiKeys = 1920;  // keys per part: 16 rows x 7.5 KiB of scores in LDS
template <int MB, bool HAS_W, int KF>  // KF: 0 bf16, 1 FP8, 2 MXFP4
__global__ __launch_bounds__(512, 1) void index_score_multi(IndexScoreArgs a, int64_t parts) {
  constexpr bool FP8 = KF == 1, FP4 = KF == 2;
  constexpr int HI = 16 * MB;
  constexpr int DI = 128;
  constexpr int KS = 4;
  constexpr int KB = FP4 ? 64 : (FP8 ? 128 : 256);  // code bytes per key
  constexpr int TB = FP4 ? kTileBytes4 : (FP8 ? kTileBytes8 : kTileBytes);
  constexpr int DEPTH = KF ? 2 * kMultiDepth : kMultiDepth;
  constexpr int NLW = FP4 ? 1 : TB / 1024;  // loading wavefronts
  constexpr int LPT = FP4 ? 2 : 1;          // loads per tile and loading wavefront
  static_assert(DEPTH <= 16, "wait_tiles covers the ring");
  __shared__ __attribute__((aligned(16))) uint8_t ring[DEPTH][TB];
  __shared__ __attribute__((aligned(16))) float sbuf[kMultiRows][kMultiKeys];
  __shared__ float sdump[64];  // stores of tiles past the end
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int64_t rblk = blockIdx.x / parts;
  const int64_t part = blockIdx.x % parts;
  const int64_t row0 = a.row0 + rblk * kMultiRows;  // first row of the block (a multiple of 16; T % 16 == 0)
  const int64_t b = row0 / a.T;
  const int64_t n_b = seq_len(a.lay, a.n_ctx, a.T, b);
  int64_t nvmax = (n_b - a.T + (row0 + kMultiRows - 1) % a.T) / a.m;  // the block's last row sees most
  if (nvmax > a.L) nvmax = a.L;
  const int64_t kb = part * kMultiKeys;
  const int64_t ke = kb + kMultiKeys < a.L ? kb + kMultiKeys : a.L;
  const int64_t kv = ke < nvmax ? ke : nvmax;
  const int ntiles = kv > kb ? static_cast<int>((kv - kb + kTileKeys - 1) / kTileKeys) : 0;
  const char* kbase = static_cast<const char*>(a.k) + b * a.L * KB;
  // MXFP4 scales follow the code bytes of all B * L keys, 4 per key.
  const char* sbase = static_cast<const char*>(a.k) + a.B * a.L * KB + b * a.L * 4;
  // load w (w < NLW) of a tile, in the streaming scan's layout.  bf16: keys
  // 4w .. 4w+3, piece p of key kk at slot p ^ kk.  FP8: keys 8w .. 8w+7,
  // piece p of key kk at slot (p + kk/2) % 8.  MXFP4: the codes (block p of
  // key kk at slot (p + kk/4) % 4), then key l%16's four scales at 1024 + 4l.
  const int kk = FP4 ? lane >> 2 : (FP8 ? 8 * (wave % NLW) + (lane >> 3) : 4 * (wave % NLW) + g);
  const uint32_t voff = FP4 ? kk * 64 + ((((lane & 3) - (kk >> 2)) & 3) << 4)
                            : (FP8 ? kk * 128 + ((((lane & 7) - (kk >> 1)) & 7) << 4) : kk * 256 + ((c16 ^ kk) << 4));
  auto issue = [&](int it) {
    uint8_t* slot = &ring[it % DEPTH][0] + (wave % NLW) * 1024;
    const int64_t t0 = kb + static_cast<int64_t>(it) * kTileKeys;
    if (t0 + kTileKeys <= a.L) {
      dma16(kbase + t0 * KB, voff, slot);
      if constexpr (FP4) dma4(sbase + t0 * 4, c16 * 4, slot + 1024);
    } else {
      int64_t s = t0 + kk;
      s = s < a.L - 1 ? s : a.L - 1;
      dma16(kbase + s * KB + (voff - kk * KB), slot);
      if constexpr (FP4) {
        int64_t s1 = t0 + c16;
        s1 = s1 < a.L - 1 ? s1 : a.L - 1;
        dma4(sbase + s1 * 4, slot + 1024);
      }
    }
  };
  if (wave < NLW) {
#pragma unroll
    for (int i = 0; i < DEPTH - 2; ++i)
      if (i < ntiles) issue(i);
  }
  bf16x8 afrag[kMultiRpw][MB][KF ? 1 : KS];
  i32x8 afrag8[kMultiRpw][MB];
  int qsc[kMultiRpw][MB];  // MXFP4: E8M0 scale of this lane's 32 query elements
  float wr[kMultiRpw][MB][HAS_W ? 4 : 1];
#pragma unroll
  for (int i = 0; i < kMultiRpw; ++i) {
    const int64_t row = row0 + kMultiRpw * wave + i;
    if constexpr (FP4) {
      const uint8_t* qb = static_cast<const uint8_t*>(a.q);
      const uint8_t* qs = qb + a.B * a.T * HI * 64;  // scales follow all code bytes
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(qb + (row * HI + mb * 16 + c16) * 64 + 16 * g);
        afrag8[i][mb] = i32x8{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]),
                              static_cast<int>(x[3]), 0, 0, 0, 0};
        qsc[i][mb] = qs[(row * HI + mb * 16 + c16) * 4 + g];
      }
    } else if constexpr (FP8) {
      const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + row * HI * DI;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        afrag8[i][mb] = *reinterpret_cast<const i32x8*>(qrow + (mb * 16 + c16) * DI + 32 * g);
    } else {
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + row * HI * DI;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          afrag[i][mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (mb * 16 + c16) * DI + ks * 32 + g * 8);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < (HAS_W ? 4 : 1); ++r) wr[i][mb][r] = HAS_W ? a.w[row * HI + mb * 16 + 4 * g + r] : 1.f;
  }
  // Two tiles per barrier: tiles it and it+1 (slots it%8, (it+1)%8); their
  // slots are refilled with tiles it+DEPTH-2 and it+DEPTH-1 after the next
  // barrier.  Software pipelined: the epilogue of a tile (ReLU, head weights,
  // head sum: VALU work that depends on its accumulators) is issued between
  // the MFMAs of the next tile rather than after them, so the matrix unit is
  // not left idle while a wavefront finishes a tile.  The last tile of a pair
  // is finished after the next barrier.  A tile past the end is computed on
  // a stale ring slot and its scores are dropped.
  using Acc = f32x4[kMultiRpw][MB];
  // The first k-step takes a zero accumulator operand (an inline constant:
  // no register clearing).
  constexpr f32x4 kZero4{0.f, 0.f, 0.f, 0.f};
  auto mfma_tile = [&](int tt, Acc& acc) {
    if constexpr (FP4) {  // key c16's code block g (rotated by c16 / 4) and its E8M0 scale (copy g)
      const uint8_t* t = &ring[tt % DEPTH][0];
      const u32x4 x = *reinterpret_cast<const u32x4*>(t + c16 * 64 + (((g + (c16 >> 2)) & 3) << 4));
      const int ksc = static_cast<int>((*reinterpret_cast<const uint32_t*>(t + 1024 + 64 * g + 4 * c16) >> (8 * g)) & 0xffu);
      const i32x8 cur4{static_cast<int>(x[0]), static_cast<int>(x[1]), static_cast<int>(x[2]), static_cast<int>(x[3]),
                       0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kMultiRpw; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)  // format 4 = E2M1 for both operands, per-lane E8M0 scales
          acc[i][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag8[i][mb], cur4, kZero4, 4, 4, 0,
                                                                        qsc[i][mb], 0, ksc);
    } else if constexpr (FP8) {  // key c16's dims 32g .. 32g+31: blocks 2g, 2g+1 (rotated by c16 / 2)
      const uint8_t* t = &ring[tt % DEPTH][0] + c16 * 128;
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(t + (((2 * g + (c16 >> 1)) & 7) << 4));
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(t + (((2 * g + 1 + (c16 >> 1)) & 7) << 4));
      const i32x8 cur8{static_cast<int>(x0[0]), static_cast<int>(x0[1]), static_cast<int>(x0[2]), static_cast<int>(x0[3]),
                       static_cast<int>(x1[0]), static_cast<int>(x1[1]), static_cast<int>(x1[2]), static_cast<int>(x1[3])};
#pragma unroll
      for (int i = 0; i < kMultiRpw; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[i][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag8[i][mb], cur8, kZero4, 0, 0, 0, 127, 0,
                                                                        127);
    } else {
      const uint8_t* t = &ring[tt % DEPTH][0] + c16 * 256;
      bf16x8 cur[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) cur[ks] = *reinterpret_cast<const bf16x8*>(t + (((4 * ks + g) ^ c16) << 4));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < kMultiRpw; ++i)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[i][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[i][mb][ks], cur[ks], ks == 0 ? kZero4 : acc[i][mb],
                                                                 0, 0, 0);
    }
  };
  // Both rows' group sums in one exchange: lane groups 0, 1 then hold row 0's
  // score and groups 2, 3 row 1's, so every lane stores one (the pairs store
  // equal values to one slot), a dropped tile to a dump slot.
  static_assert(kMultiRpw == 2, "two rows per wavefront share the group sums");
  auto epi_tile = [&](int tt, bool keep, const Acc& acc) {
    const float tot = group_sum4_pair(head_part<MB, HAS_W>(acc[0], wr[0]), head_part<MB, HAS_W>(acc[1], wr[1]));
    float* dst = keep ? &sbuf[kMultiRpw * wave + (g >> 1)][(keep ? tt : 0) * kTileKeys + c16] : &sdump[lane];
    *dst = tot;
  };
  // Interleave n MFMAs with the VALU work around them, m VALU per MFMA.
  auto interleave = [](auto n, auto m) {
#pragma unroll
    for (int q = 0; q < decltype(n)::value; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(m)::value, 0);
    }
  };
  using NM = std::integral_constant<int, kMultiRpw * MB * (KF ? 1 : KS)>;  // MFMAs per tile
  using NV = std::integral_constant<int, (MB * 8 + 6) * kMultiRpw / (kMultiRpw * MB * (KF ? 1 : KS)) + 1>;
  Acc accp;  // the previous pair's second tile, finished after this barrier (then reused for this pair's)
  int ttp = -1;
#pragma unroll
  for (int i = 0; i < kMultiRpw; ++i)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) accp[i][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < ntiles; it += 2) {
    if (wave < NLW) {
      // loads issued after tile it+1's (or it's, at the end) may stay in flight
      const int last = it + 1 < ntiles ? it + 1 : it;
      const int issued = it + DEPTH - 2 < ntiles ? it + DEPTH - 2 : ntiles;  // tiles [0, issued) issued
      wait_tiles<LPT>(issued - 1 - last);
    }
    __syncthreads();  // tiles it, it+1 in LDS; every wave is done with it-2, it-1
    if (wave < NLW) {
      if (it + DEPTH - 2 < ntiles) issue(it + DEPTH - 2);  // into tile it-2's slot
      if (it + DEPTH - 1 < ntiles) issue(it + DEPTH - 1);  // into tile it-1's slot
    }
    Acc acc0;
    mfma_tile(it, acc0);
    epi_tile(ttp, ttp >= 0, accp);
    interleave(NM{}, NV{});
    mfma_tile(it + 1, accp);
    epi_tile(it, true, acc0);
    interleave(NM{}, NV{});
    ttp = it + 1 < ntiles ? it + 1 : -1;
  }
  epi_tile(ttp, ttp >= 0, accp);
  // this wave's rows, keys [kb, ke): computed and visible, else -inf
  const int nk = static_cast<int>(ke - kb);
  const int nc = ntiles * kTileKeys;
#pragma unroll
  for (int i = 0; i < kMultiRpw; ++i) {
    const int64_t row = row0 + kMultiRpw * wave + i;
    int64_t nv = (n_b - a.T + row % a.T) / a.m;
    if (nv > a.L) nv = a.L;
    float* srow = a.score + (row - a.row0) * a.ld;
    const float* sb = sbuf[kMultiRpw * wave + i];
    for (int o = lane; o < nk; o += 64) srow[kb + o] = (o < nc && kb + o < nv) ? sb[o] : -INFINITY;
  }
}

// Other d_I (64): MFMA operands straight from global memory (64 B per key
// per load instruction).
template <int MB, int KS, bool HAS_W>
__global__ __launch_bounds__(256) void index_score_mfma_direct(IndexScoreArgs a, int64_t parts) {
  constexpr int HI = 16 * MB;
  constexpr int DI = 32 * KS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t lrow = blockIdx.x / parts;
  const int64_t part = blockIdx.x % parts;
  const int64_t row = a.row0 + lrow;
  const int64_t b = row / a.T;
  const int64_t tpos = seq_len(a.lay, a.n_ctx, a.T, b) - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  float* srow = a.score + lrow * a.ld;
  const int64_t wave_begin = part * kDirectKeysPerWg + wave * (kDirectTiles * kTileKeys);
  if (wave_begin >= a.L) return;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + g * 8;
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + row * HI * DI;
  bf16x8 afrag[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      afrag[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (mb * 16 + c16) * DI + ks * 32 + g * 8);
  for (int it = 0; it < kDirectTiles; ++it) {
    int64_t s = wave_begin + it * kTileKeys + c16;
    const int64_t sc = s < a.L - 1 ? s : a.L - 1;
    bf16x8 cur[KS];
    const int64_t kr = cache_row(a.lay, a.L, b, sc);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cur[ks] = *reinterpret_cast<const bf16x8*>(kbase + kr * DI + ks * 32);
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[mb][ks], cur[ks], acc[mb], 0, 0, 0);
    float part_sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rl = relu_bits(acc[mb][r]);
        part_sum = HAS_W ? fmaf(a.w[row * HI + mb * 16 + 4 * g + r], rl, part_sum) : part_sum + rl;
      }
    part_sum += __shfl_xor(part_sum, 16, 64);
    part_sum += __shfl_xor(part_sum, 32, 64);
    const float val = s < nv ? part_sum : -INFINITY;
    if (g == 0 && s < a.L) srow[s] = val;
  }
}

// fp32 storage: VALU dot products in fp32 (small indexer shapes).
__global__ __launch_bounds__(256) void index_score_f32(IndexScoreArgs a, int64_t parts) {
  extern __shared__ float qs[];
  const int64_t lrow = blockIdx.x / parts;
  const int64_t part = blockIdx.x % parts;
  const int64_t row = a.row0 + lrow;
  const int64_t b = row / a.T;
  const int64_t tpos = seq_len(a.lay, a.n_ctx, a.T, b) - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  const float* q = static_cast<const float*>(a.q) + row * a.HI * a.dI;
  for (int64_t i = threadIdx.x; i < a.HI * a.dI; i += blockDim.x) qs[i] = q[i];
  __syncthreads();
  const int64_t s = part * blockDim.x + threadIdx.x;
  if (s >= a.L) return;
  float* srow = a.score + lrow * a.ld;
  if (s >= nv) {
    srow[s] = -INFINITY;
    return;
  }
  const float* kr = static_cast<const float*>(a.k) + cache_row(a.lay, a.L, b, s) * a.dI;
  float tot = 0.f;
  for (int64_t h = 0; h < a.HI; ++h) {
    float dot = 0.f;
    for (int64_t c = 0; c < a.dI; ++c) dot = fmaf(qs[h * a.dI + c], kr[c], dot);
    const float wh = a.w ? a.w[row * a.HI + h] : 1.0f;
    tot = fmaf(wh, fmaxf(dot, 0.f), tot);
  }
  srow[s] = tot;
}

}  // namespace

void index_plan(int64_t nrows, int64_t L, int64_t* parts_out, int64_t* per_wave_out) {
  // About one workgroup per CU in one round; every wavefront streams
  // kMinKeysPerWave .. kMaxKeysPerWave keys.
  const int64_t target = 256;
  int64_t parts = (target + nrows - 1) / nrows;
  int64_t per_wave = (L + kWaves * parts - 1) / (kWaves * parts);
  per_wave = (per_wave + kTileKeys - 1) / kTileKeys * kTileKeys;
  if (per_wave < kMinKeysPerWave) per_wave = kMinKeysPerWave;
  if (per_wave > kMaxKeysPerWave) per_wave = kMaxKeysPerWave;
  *parts_out = (L + kWaves * per_wave - 1) / (kWaves * per_wave);
  *per_wave_out = per_wave;
}

namespace {

// Timing request for the next streaming scan launched by this host thread:
// its kernel records these events as it starts and ends (hipExtLaunchKernel
// stamps the dispatch itself, so no event packet sits between kernels).
thread_local hipEvent_t t_scan_start = nullptr, t_scan_stop = nullptr;

template <typename K>
void launch_scan_kernel(K kern, dim3 grid, dim3 block, hipStream_t s, const IndexScoreArgs& a, int64_t parts,
                        int64_t per_wave, const IndexCandidates& co) {
  if (t_scan_start != nullptr && t_scan_stop != nullptr) {
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, t_scan_start, t_scan_stop, 0, a, parts, per_wave, co);
    t_scan_start = t_scan_stop = nullptr;
  } else {
    hipLaunchKernelGGL(kern, grid, block, 0, s, a, parts, per_wave, co);
  }
}

template <bool TOPK>
hipError_t launch_stream(const IndexScoreArgs& a, const IndexCandidates& co, hipStream_t s) {
  int64_t parts, per_wave;
  index_plan(a.nrows, a.L, &parts, &per_wave);
  const dim3 grid(static_cast<uint32_t>(a.nrows * parts));
  const int mb = static_cast<int>(a.HI / 16);
  const bool w = a.w != nullptr;
  const int kf = a.dt == kMXFP4 ? 2 : (a.dt == kFP8 ? 1 : 0);
#define CSA_INDEX_KF(MB_, KF_)                                                                                    \
  if (w) launch_scan_kernel(index_score_stream<MB_, true, TOPK, KF_>, grid, dim3(KF_ ? 64 * kWaves8 : 256), s, a,   \
                            parts, per_wave, co);                                                                    \
  else launch_scan_kernel(index_score_stream<MB_, false, TOPK, KF_>, grid, dim3(KF_ ? 64 * kWaves8 : 256), s, a,    \
                          parts, per_wave, co);
#define CSA_INDEX_LAUNCH(MB_)                  \
  case MB_:                                    \
    if (kf == 2) { CSA_INDEX_KF(MB_, 2) }      \
    else if (kf == 1) { CSA_INDEX_KF(MB_, 1) } \
    else { CSA_INDEX_KF(MB_, 0) }              \
    break;
  switch (mb) {
    CSA_INDEX_LAUNCH(1)
    CSA_INDEX_LAUNCH(2)
    CSA_INDEX_LAUNCH(4)
    CSA_INDEX_LAUNCH(8)
    default: return hipErrorInvalidValue;
  }
#undef CSA_INDEX_LAUNCH
#undef CSA_INDEX_KF
  return hipGetLastError();
}

}  // namespace

void time_next_scan(hipEvent_t start, hipEvent_t stop) {
  t_scan_start = start;
  t_scan_stop = stop;
}

hipError_t launch_index_score(const IndexScoreArgs& a, hipStream_t s) {
  if (a.nrows == 0 || a.L == 0) return hipSuccess;
  const int mb = static_cast<int>(a.HI / 16), ks = static_cast<int>(a.dI / 32);
  const bool w = a.w != nullptr;
  // Many query rows of one sequence (prefill), bf16, FP8 or MXFP4 keys in
  // dense caches: the 16-row kernel reads each key tile once per 16 rows.
  if ((a.dt == kBF16 || a.dt == kFP8 || a.dt == kMXFP4) && ks == 4 && !a.lay.bt &&
      index_multi_rows(a.T, a.HI, a.row0, a.nrows)) {
    const int64_t parts = (a.L + kMultiKeys - 1) / kMultiKeys;
    const dim3 grid(static_cast<uint32_t>(a.nrows / kMultiRows * parts));
    const dim3 block(64 * kMultiRows / kMultiRpw);
    const int kf = a.dt == kMXFP4 ? 2 : (a.dt == kFP8 ? 1 : 0);
#define CSA_INDEX_MULTI_KF(MB_, KF_)                                                                \
  if (w) hipLaunchKernelGGL((index_score_multi<MB_, true, KF_>), grid, block, 0, s, a, parts);       \
  else hipLaunchKernelGGL((index_score_multi<MB_, false, KF_>), grid, block, 0, s, a, parts);
#define CSA_INDEX_MULTI(MB_)                            \
  case MB_:                                             \
    if (kf == 2) { CSA_INDEX_MULTI_KF(MB_, 2) }         \
    else if (kf == 1) { CSA_INDEX_MULTI_KF(MB_, 1) }    \
    else { CSA_INDEX_MULTI_KF(MB_, 0) }                 \
    break;
    switch (mb) {
      CSA_INDEX_MULTI(1)
      CSA_INDEX_MULTI(2)
      CSA_INDEX_MULTI(4)
      default: return hipErrorInvalidValue;
    }
#undef CSA_INDEX_MULTI
#undef CSA_INDEX_MULTI_KF
    return hipGetLastError();
  }
  if (a.dt == kFP8 || a.dt == kMXFP4) {  // d_I = 128 only (index_shape_supported)
    if (a.dI != 128) return hipErrorInvalidValue;
    return launch_stream<false>(a, IndexCandidates{}, s);
  }
  if (a.dt == kBF16) {
    if (ks == 4) return launch_stream<false>(a, IndexCandidates{}, s);
    if (ks == 2) {
      const int64_t parts = (a.L + kDirectKeysPerWg - 1) / kDirectKeysPerWg;
      const dim3 grid(static_cast<uint32_t>(a.nrows * parts));
#define CSA_INDEX_LAUNCH(MB_)                                                                             \
  case MB_:                                                                                               \
    if (w) hipLaunchKernelGGL((index_score_mfma_direct<MB_, 2, true>), grid, dim3(256), 0, s, a, parts);  \
    else hipLaunchKernelGGL((index_score_mfma_direct<MB_, 2, false>), grid, dim3(256), 0, s, a, parts);   \
    break;
      switch (mb) {
        CSA_INDEX_LAUNCH(2)
        CSA_INDEX_LAUNCH(4)
        default: return hipErrorInvalidValue;
      }
#undef CSA_INDEX_LAUNCH
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  const int64_t parts = (a.L + 255) / 256;
  const size_t lds = static_cast<size_t>(a.HI * a.dI) * sizeof(float);
  hipLaunchKernelGGL(index_score_f32, dim3(static_cast<uint32_t>(a.nrows * parts)), dim3(256), lds, s, a, parts);
  return hipGetLastError();
}

bool index_multi_rows(int64_t T, int64_t HI, int64_t row0, int64_t nrows) {
  // H_I <= 64: two rows' query blocks stay in registers
  return HI <= 64 && HI % 16 == 0 && T >= 64 && T % kMultiRows == 0 && row0 % kMultiRows == 0 &&
         nrows % kMultiRows == 0 && nrows > 0;
}

bool index_topk_fusable(int64_t nrows, int64_t L, int64_t HI, int64_t dI, int64_t k, Dt dt) {
  if ((dt != kBF16 && dt != kFP8 && dt != kMXFP4) || dI != 128 || nrows <= 0 || L <= 0 || k < 1 || k > kCandStage)
    return false;
  if (!(HI == 16 || HI == 32 || HI == 64 || HI == 128)) return false;
  int64_t parts, per_wave;
  index_plan(nrows, L, &parts, &per_wave);
  return parts <= 256 && parts * k <= 16384;
}

// Workspace of the fused path: per (row, part) the top-k candidates (8 B
// each) and their count, then the compact lists (8 B per entry) with their
// count and threshold.
size_t index_topk_fused_ws_bytes(int64_t nrows, int64_t L, int64_t k) {
  int64_t parts, per_wave, lrank, lcap;
  index_plan(nrows, L, &parts, &per_wave);
  compact_list_plan(parts, k, &lrank, &lcap);
  const size_t units = static_cast<size_t>(nrows) * parts;
  const size_t b = units * (static_cast<size_t>(k) * 8 + 4) + units * (static_cast<size_t>(lcap) * 8 + 8);
  return (b + 255) / 256 * 256;
}

hipError_t launch_index_topk_fused(const IndexScoreArgs& a, const TopkArgs& t, void* ws, hipStream_t s) {
  if (a.nrows == 0) return hipSuccess;
  int64_t parts, per_wave;
  index_plan(a.nrows, a.L, &parts, &per_wave);
  const int64_t units = a.nrows * parts;
  IndexCandidates co;
  co.cap = t.k;
  co.cval = static_cast<float*>(ws);
  co.cidx = reinterpret_cast<int32_t*>(co.cval + units * t.k);
  co.ccnt = co.cidx + units * t.k;
  compact_list_plan(parts, t.k, &co.lrank, &co.lcap);
  if (co.lrank > 0) {
    co.lval = reinterpret_cast<float*>(co.ccnt + units);
    co.lidx = reinterpret_cast<int32_t*>(co.lval + units * co.lcap);
    co.lcnt = co.lidx + units * co.lcap;
    co.lthr = reinterpret_cast<float*>(co.lcnt + units);
  }
  const hipError_t e = launch_stream<true>(a, co, s);
  if (e != hipSuccess) return e;
  return launch_topk_merge(t, parts, co, true, s);
}

// Listed path geometry: r = kMergeUnion / parts (at least twice a part's
// share k / parts of the row's top-k, so that a part rarely holds more than
// its list), list capacity 2r for ties.
static void listed_plan(int64_t nrows, int64_t L, int64_t k, int64_t* parts, int64_t* r) {
  int64_t per_wave;
  index_plan(nrows, L, parts, &per_wave);
  *r = kMergeUnion / *parts;
  if (kWaves * per_wave > kListPartKeysMax || *parts > 512 || *r * *parts < k || *r < 2 * ((k + *parts - 1) / *parts) ||
      2 * k > mrg::kStage)
    *r = 0;
}

bool index_topk_listable(int64_t nrows, int64_t L, int64_t HI, int64_t dI, int64_t k, Dt dt) {
  if ((dt != kBF16 && dt != kFP8 && dt != kMXFP4) || dI != 128 || nrows <= 0 || L <= 0 || k < 1) return false;
  if (!(HI == 16 || HI == 32 || HI == 64 || HI == 128)) return false;
  int64_t parts, r;
  listed_plan(nrows, L, k, &parts, &r);
  return r > 0;
}

// Workspace of the listed path: the scores [nrows][L], the stand-alone
// top-k's state for every row (the fallback), then per (row, part) a list of
// 2r entries (8 B each), its count and threshold, then one flag per row.
static size_t align256(size_t b) { return (b + 255) / 256 * 256; }
size_t index_topk_listed_ws_bytes(int64_t nrows, int64_t L, int64_t k) {
  int64_t parts, r;
  listed_plan(nrows, L, k, &parts, &r);
  if (r == 0) return 0;  // not a listed shape
  const size_t units = static_cast<size_t>(nrows) * parts;
  return align256(static_cast<size_t>(nrows) * L * sizeof(float)) + nrows * topk_ws_bytes_per_row(L, k) +
         align256(units * (2 * r * 8 + 8)) + align256(static_cast<size_t>(nrows) * 4);
}

hipError_t launch_index_topk_listed(const IndexScoreArgs& a0, const TopkArgs& t0, void* ws, hipStream_t s) {
  if (a0.nrows == 0) return hipSuccess;
  int64_t parts, r;
  listed_plan(a0.nrows, a0.L, t0.k, &parts, &r);
  if (r == 0) return hipErrorInvalidValue;
  const int64_t units = a0.nrows * parts;
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* sc = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(a0.nrows) * a0.L * sizeof(float));
  void* sel_ws = p;
  p += a0.nrows * topk_ws_bytes_per_row(a0.L, t0.k);
  IndexCandidates co;
  co.cap = 0;
  co.cval = nullptr;
  co.cidx = nullptr;
  co.ccnt = nullptr;
  co.lrank = r;
  co.lcap = 2 * r;
  co.lval = reinterpret_cast<float*>(p);
  co.lidx = reinterpret_cast<int32_t*>(co.lval + units * co.lcap);
  co.lcnt = co.lidx + units * co.lcap;
  co.lthr = reinterpret_cast<float*>(co.lcnt + units);
  p += align256(static_cast<size_t>(units) * (2 * r * 8 + 8));
  int32_t* done = reinterpret_cast<int32_t*>(p);
  IndexScoreArgs a = a0;
  a.score = sc;
  a.ld = a0.L;
  a.row0 = 0;
  hipError_t e = launch_stream<false>(a, co, s);
  if (e != hipSuccess) return e;
  TopkArgs t = t0;
  t.score = sc;
  t.ld = a0.L;
  t.row0 = 0;
  e = launch_topk_list_merge(t, parts, co, done, s);
  if (e != hipSuccess) return e;
  t.done = done;
  return launch_topk(t, sel_ws, s);  // rows the lists did not settle
}

bool index_shape_supported(int64_t HI, int64_t dI, Dt dt) {
  if (dt == kFP8 || dt == kMXFP4) return dI == 128 && (HI == 16 || HI == 32 || HI == 64 || HI == 128);
  if (dt == kF32) return HI * dI * 4 <= 65536;
  if (HI % 16 || dI % 32) return false;
  const int64_t mb = HI / 16, ks = dI / 32;
  return (ks == 4 && (mb == 1 || mb == 2 || mb == 4 || mb == 8)) || (ks == 2 && (mb == 2 || mb == 4));
}

}  // namespace csa
