// Top-k selection over indexer scores: per query keep the min(k, |V_t|)
// highest scores among the visible entries, equal scores going to the lower
// entry index; write the kept indices in ascending order, -1 padded.
//
// Method: shareware.cn Hybrid Attention article, section 六 (score the
// compressed entries, keep the top-k candidates for the main attention);
// aimodeling.com news item, CSA paragraph (1024 entries per query).
//
// Design (gfx950): exact radix select on order-preserving 32-bit keys
// (-0 and +0 share a key, so they tie), in two launches so that a decode row
// of 250K scores is spread over many workgroups:
//   1. part kernel: the row is cut into parts of 16384 scores; one 512-thread
//      workgroup holds a part in registers (32 consecutive entries per
//      thread, loaded 16 bytes at a time), selects the part's own
//      top-min(k, part) with LDS histogram passes of up to 11 bits that start
//      below the common bit prefix of the part's keys, and writes the kept
//      (score, index) pairs in index order.  Any entry of the row's top-k is
//      in its part's top-k, ties included, because fewer entries beat it
//      inside the part than in the whole row.
//   2. merge kernel: one workgroup per row runs the same selection over the
//      concatenated part candidates (part order = index order) and compacts
//      the winners in order.
//   A third kernel serves the listed index path: one workgroup per row merges
//   the exact short lists the scan wrote for its key ranges and flags the
//   rows they settle; the two kernels above then return at once for those.
// Latency, not bandwidth, bounds both (a part is 64 KiB), so each histogram
// pass costs three barriers (double-buffered bins, wave scans), and the
// ordered compaction is one 32-bit workgroup scan of per-thread (greater,
// equal) counts packed in 16-bit halves, which makes the lower-index tie rule
// exact without a sort.
#include "common.hpp"
#include "kernels.hpp"
#include "merge.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kThreads = 512;
constexpr int kItems = 32;
constexpr int64_t kPart = static_cast<int64_t>(kThreads) * kItems;  // 16384
constexpr int kBins = sel::kBins;
constexpr int kMaxMergeParts = 256;  // one part count per merge thread
constexpr int kStage = mrg::kStage;  // outputs up to this size are staged in LDS, then stored coalesced
using Sel = sel::Select<kThreads, kItems>;
using sel::lane_id;
using sel::wave_incl_scan;

// Part kernel state for parts of kThreads * IT scores.
template <int IT>
struct PartShared {
  typename sel::Filter<kThreads, IT, 16>::Shared fs;
  int32_t si[kStage + 64];  // staged output: entry and score (64 lane-private dump slots at the end)
  float sv[kStage + 64];
  alignas(16) float stage[mrg::Tile<kThreads, IT>::kFloats];
};
// Half-size parts (8192 scores, 16 per thread) for launches whose candidates
// still fit the merge's tile: a workgroup then holds ~78 KiB of LDS and at
// most 128 VGPRs, so two share a CU, and each selection has half the items.
constexpr int kItemsHalf = 16;
constexpr int64_t kPartHalf = static_cast<int64_t>(kThreads) * kItemsHalf;  // 8192
static_assert(2 * sizeof(PartShared<kItemsHalf>) <= 160 * 1024, "two half-size part workgroups share a CU");

// The merge: 512 threads, 32 candidate slots each (1024 x 16 measured slower:
// more waves per barrier, no less latency per phase).
constexpr int kMThreads = 512;
using Merge = mrg::Merge<kMThreads>;
static_assert(Merge::ITEMS * kMThreads == kPart, "merge tile");
using mrg::row_visible;

// Stage 1: per-part local selection over parts of P = kThreads * IT scores.
template <int IT>
__global__ __launch_bounds__(kThreads, IT == kItemsHalf ? 2 : 1) void topk_part_kernel(TopkArgs a, int64_t nparts,
                                                                                      int64_t cap, float* cval,
                                                                                      int32_t* cidx, int32_t* ccnt) {
  using Filt = sel::Filter<kThreads, IT, 16>;
  using PartTile = mrg::Tile<kThreads, IT>;
  constexpr int64_t kPart = static_cast<int64_t>(kThreads) * IT;
  __shared__ PartShared<IT> sh;
  const int64_t lrow = blockIdx.x / nparts;
  const int64_t part = blockIdx.x % nparts;
  if (a.done && a.done[lrow]) return;  // settled by the list merge
  const int64_t nv = row_visible(a, a.row0 + lrow);
  if (nv <= a.k) return;  // the merge kernel keeps every visible entry
  const int64_t base = part * kPart;
  int64_t cnt = nv - base;
  if (cnt > kPart) cnt = kPart;
  int32_t* cc = ccnt + lrow * nparts + part;
  float* ov = cval + (lrow * nparts + part) * cap;
  int32_t* oi = cidx + (lrow * nparts + part) * cap;
  const int tid = threadIdx.x;
  if (cnt <= 0) {  // no candidate: every slot NaN
    for (int64_t i = tid; i < cap; i += kThreads) ov[i] = __builtin_nanf("");
    if (tid == 0) *cc = 0;
    return;
  }
  Filt::zero(sh.fs);
  const float* s = a.score + lrow * a.ld + base;
  float v[IT];
  PartTile::store(PartTile::load(s, static_cast<int>(cnt)), sh.stage, v);
  const int i0 = tid * IT;  // this thread's entries i0 .. i0+IT-1 of the part
  if (cnt <= cap) {  // the whole part is kept; slots past it hold NaN
    for (int64_t i = tid; i < cap; i += kThreads) {
      const float t = sh.stage[PartTile::pos(static_cast<int>(i < kPart ? i : 0))];
      ov[i] = i < cnt ? t : __builtin_nanf("");
      if (i < cnt) oi[i] = static_cast<int32_t>(base + i);
    }
    if (tid == 0) *cc = static_cast<int32_t>(cnt);
    return;
  }
  float vmin, vmax;
  Filt::block_range(v, sh.fs, &vmin, &vmax);
  const uint32_t ncnt = static_cast<uint32_t>(cnt), ucap = static_cast<uint32_t>(cap);
  auto src = [&](uint32_t e) { return sh.stage[PartTile::pos(static_cast<int>(e))]; };
  if (cap <= kStage) {  // stage the kept entries in LDS, then store them coalesced
    Filt::run(
        v, src, ncnt, ucap, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t e) {
          const uint32_t p = pos != sel::kNoSlot ? pos : kStage + lane_id();
          sh.si[p] = static_cast<int>(e);
          sh.sv[p] = val;
        },
        [&](int j, uint32_t pos) {
          sh.si[pos] = i0 + j;
          sh.sv[pos] = sh.stage[PartTile::pos(i0 + j)];
        });
    for (int i = tid; i < cap; i += kThreads) {
      ov[i] = sh.sv[i];
      oi[i] = static_cast<int32_t>(base + sh.si[i]);
    }
  } else {
    Filt::run(
        v, src, ncnt, ucap, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t e) {
          if (pos == sel::kNoSlot) return;
          ov[pos] = val;
          oi[pos] = static_cast<int32_t>(base + e);
        },
        [&](int j, uint32_t pos) {
          ov[pos] = sh.stage[PartTile::pos(i0 + j)];
          oi[pos] = static_cast<int32_t>(base + i0 + j);
        });
  }
  if (tid == 0) *cc = static_cast<int32_t>(cap);
}

// Stage 2: per-row merge of the part candidates.  Rows with at most k
// visible entries keep all of them (the part kernel skipped them).
__device__ __forceinline__ bool merge_trivial(const TopkArgs& a, int64_t lrow) {
  const int64_t nv = row_visible(a, a.row0 + lrow);
  if (nv > a.k) return false;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const float* s = a.score + lrow * a.ld;
  for (int64_t i = threadIdx.x; i < a.k; i += blockDim.x) {
    o[i] = i < nv ? static_cast<int32_t>(i) : -1;
    if (os) os[i] = i < nv ? s[i] : -INFINITY;
  }
  return true;
}

// Fast merge: nparts * cap <= 16384 slots and nparts <= 256, from the
// parts' compact lists when they settle the row, else from all candidates.
__global__ __launch_bounds__(kMThreads) void topk_merge_kernel(TopkArgs a, int nparts, IndexCandidates c,
                                                               bool fused) {
  __shared__ Merge::Shared sh;
  const int64_t lrow = blockIdx.x;
  if (a.done && a.done[lrow]) return;  // settled by the list merge
  if (!fused && merge_trivial(a, lrow)) return;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int k = static_cast<int>(a.k);
  const int64_t u0 = lrow * nparts;
  const int cap = static_cast<int>(c.cap);
  if (c.lval && Merge::lists<mrg::kSlots / 4 / kMThreads>(k, nparts, c.lval + u0 * c.lcap, c.lidx + u0 * c.lcap,
                                                          c.lcnt + u0, c.lthr + u0, c.lcap, sh, o, os,
                                                          c.cval + u0 * cap, c.cidx + u0 * cap, c.ccnt + u0, cap))
    return;
  // Without short lists the parts' top-k lists serve as the lists when their
  // union fits (each is its part's whole candidate set, so nothing is left
  // to test): one selection over at most a quarter of the tile.  The
  // full-tile path samples a threshold only when k is at most a quarter of
  // the valid candidates, so two parts of k each would take its radix path.
  if (!c.lval && static_cast<int64_t>(nparts) * cap <= mrg::kSlots / 4 &&
      Merge::lists<mrg::kSlots / 4 / kMThreads>(k, nparts, c.cval + u0 * cap, c.cidx + u0 * cap, c.ccnt + u0,
                                                nullptr, cap, sh, o, os))
    return;
  Merge::full(k, nparts, cap, c.cval + u0 * cap, c.cidx + u0 * cap, c.ccnt + u0, sh, o, os);
}

// List merge of the listed path: the union of the parts' exact lists settles
// the row when every part's threshold is at most the union's k-th largest
// (then the output is written and done[row] set); otherwise done[row] is
// cleared and the stand-alone top-k runs on the row's scores.  Rows with at
// most k visible entries keep all of them here.
__global__ __launch_bounds__(kMThreads) void topk_list_merge_kernel(TopkArgs a, int nparts, IndexCandidates c,
                                                                    int32_t* done) {
  __shared__ Merge::Shared sh;
  const int64_t lrow = blockIdx.x;
  bool ok = merge_trivial(a, lrow);
  if (!ok) {
    const int64_t u0 = lrow * nparts;
    ok = Merge::lists<mrg::kSlots / 4 / kMThreads>(static_cast<int>(a.k), nparts, c.lval + u0 * c.lcap,
                                                   c.lidx + u0 * c.lcap, c.lcnt + u0, c.lthr + u0, c.lcap, sh,
                                                   a.idx + lrow * a.k,
                                                   a.out_score ? a.out_score + lrow * a.k : nullptr);
  }
  if (threadIdx.x == 0) done[lrow] = ok ? 1 : 0;
}

// General merge (k >= 16384, or more than 256 parts): histogram passes over
// the slots in L2, then ordered compaction tile by tile.
__global__ __launch_bounds__(kThreads) void topk_merge_general(TopkArgs a, int64_t nparts, int64_t cap,
                                                               const float* cval, const int32_t* cidx,
                                                               const int32_t* ccnt) {
  __shared__ struct { Sel::Shared core; } sh;
  const int64_t lrow = blockIdx.x;
  if (a.done && a.done[lrow]) return;  // settled by the list merge
  if (merge_trivial(a, lrow)) return;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;
  const int64_t nslots = nparts * cap;
  const float* rv = cval + lrow * nparts * cap;
  const int32_t* ri = cidx + lrow * nparts * cap;
  const int32_t* rc = ccnt + lrow * nparts;
  Sel::zero(sh.core);
  __syncthreads();
  auto slot_ok = [&](int64_t sl) {
    const int64_t p = sl / cap;
    return sl < nslots && sl - p * cap < rc[p];
  };
  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(a.k);
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    uint32_t* h = sh.core.hist[pass & 1];
    for (int64_t sl = tid; sl < nslots; sl += kThreads) {
      if (!slot_ok(sl)) continue;
      const uint32_t key = float_key(rv[sl]);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1u);
    }
    for (int i = tid; i < kBins; i += kThreads) sh.core.hist[(pass & 1) ^ 1][i] = 0;
    __syncthreads();
    constexpr int kBpt = kBins / kThreads;
    uint32_t c[kBpt], s = 0;
#pragma unroll
    for (int q = 0; q < kBpt; ++q) {
      const int bq = nb - 1 - kBpt * tid - q;
      c[q] = bq >= 0 ? h[bq] : 0u;
      s += c[q];
    }
    const uint32_t incl = wave_incl_scan(s);
    if (lane_id() == 63) sh.core.wsum[tid >> 6] = incl;
    __syncthreads();
    uint32_t excl = incl - s;
    for (int w = 0; w < (tid >> 6); ++w) excl += sh.core.wsum[w];
#pragma unroll
    for (int q = 0; q < kBpt; ++q) {
      const int bq = nb - 1 - kBpt * tid - q;
      if (bq >= 0 && excl < remaining && excl + c[q] >= remaining) {
        sh.core.sel_bin = static_cast<uint32_t>(bq);
        sh.core.sel_above = excl;
      }
      excl += c[q];
    }
    __syncthreads();
    prefix |= sh.core.sel_bin << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    remaining -= sh.core.sel_above;
  }
  uint32_t bg = 0, be = 0;
  for (int64_t t0 = 0; t0 < nslots; t0 += kPart) {
    uint32_t keys[kItems];
    float v[kItems];
    int32_t ix[kItems];
    uint32_t vmask = 0;
    for (int j = 0; j < kItems; ++j) {
      const int64_t sl = t0 + static_cast<int64_t>(tid) * kItems + j;
      const bool ok = slot_ok(sl);
      vmask |= static_cast<uint32_t>(ok) << j;
      v[j] = ok ? rv[sl] : 0.f;
      ix[j] = ok ? ri[sl] : 0;
      keys[j] = float_key(v[j]);
    }
    const int64_t sl0 = t0 + static_cast<int64_t>(tid) * kItems;
    Sel::compact(keys, vmask, prefix, remaining, sh.core, &bg, &be, [&](int j, uint32_t pos) {
      o[pos] = ri[sl0 + j];
      if (os) os[pos] = rv[sl0 + j];
    });
  }
}

}  // namespace

int64_t topk_cap(int64_t k) { return k < kPart ? k : kPart; }
// Half-size parts when their candidates fit the merge's tile and k is at most
// a quarter of a part (the sampled selection's range); else 16384-score parts.
bool topk_half_parts(int64_t L, int64_t k) {
  const int64_t np = L <= 0 ? 1 : (L + kPartHalf - 1) / kPartHalf;
  return 4 * k <= kPartHalf && np * topk_cap(k) <= kPart && np <= kMaxMergeParts;
}
int64_t topk_parts(int64_t L, int64_t k) {
  const int64_t ps = topk_half_parts(L, k) ? kPartHalf : kPart;
  return L <= 0 ? 1 : (L + ps - 1) / ps;
}

size_t topk_ws_bytes_per_row(int64_t L, int64_t k) {
  const int64_t np = topk_parts(L, k);
  const size_t b = static_cast<size_t>(np) * topk_cap(k) * 8 + static_cast<size_t>(np) * 4;
  return (b + 255) / 256 * 256;
}

hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t s) {
  if (a.nrows == 0 || a.k == 0) return hipSuccess;
  const int64_t np = topk_parts(a.L, a.k), cap = topk_cap(a.k);
  float* cval = static_cast<float*>(ws);
  int32_t* cidx = reinterpret_cast<int32_t*>(cval + a.nrows * np * cap);
  int32_t* ccnt = cidx + a.nrows * np * cap;
  if (topk_half_parts(a.L, a.k))
    hipLaunchKernelGGL(topk_part_kernel<kItemsHalf>, dim3(static_cast<uint32_t>(a.nrows * np)), dim3(kThreads), 0, s,
                       a, np, cap, cval, cidx, ccnt);
  else
    hipLaunchKernelGGL(topk_part_kernel<kItems>, dim3(static_cast<uint32_t>(a.nrows * np)), dim3(kThreads), 0, s, a,
                       np, cap, cval, cidx, ccnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  IndexCandidates c;
  c.cval = cval;
  c.cidx = cidx;
  c.ccnt = ccnt;
  c.cap = cap;
  return launch_topk_merge(a, np, c, false, s);
}

hipError_t launch_topk_list_merge(const TopkArgs& a, int64_t np, const IndexCandidates& c, int32_t* done,
                                  hipStream_t s) {
  if (a.nrows == 0 || a.k == 0) return hipSuccess;
  if (np > kMThreads || 2 * a.k > kStage) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_list_merge_kernel, dim3(static_cast<uint32_t>(a.nrows)), dim3(kMThreads), 0, s, a,
                     static_cast<int>(np), c, done);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const TopkArgs& a, int64_t np, const IndexCandidates& c, bool fused, hipStream_t s) {
  if (a.nrows == 0 || a.k == 0) return hipSuccess;
  if (np * c.cap <= kPart && np <= kMaxMergeParts) {
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<uint32_t>(a.nrows)), dim3(kMThreads), 0, s, a,
                       static_cast<int>(np), c, fused);
  } else {
    if (fused) return hipErrorInvalidValue;  // the fused path only takes the fast merge
    hipLaunchKernelGGL(topk_merge_general, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a, np, c.cap,
                       c.cval, c.cidx, c.ccnt);
  }
  return hipGetLastError();
}

}  // namespace csa
