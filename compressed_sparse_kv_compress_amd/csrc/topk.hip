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
// Latency, not bandwidth, bounds both (a part is 64 KiB), so each histogram
// pass costs three barriers (double-buffered bins, wave scans), and the
// ordered compaction is one 32-bit workgroup scan of per-thread (greater,
// equal) counts packed in 16-bit halves, which makes the lower-index tie rule
// exact without a sort.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kThreads = 512;
constexpr int kItems = 32;
constexpr int64_t kPart = static_cast<int64_t>(kThreads) * kItems;  // 16384
constexpr int kBins = sel::kBins;
constexpr int kMaxMergeParts = 256;  // one part count per merge thread
constexpr int kStage = 2048;         // outputs up to this size are staged in LDS, then stored coalesced
using Sel = sel::Select<kThreads, kItems>;
using Filt = sel::Filter<kThreads, kItems, 16>;
using sel::lane_id;
using sel::wave_incl_scan;

// A tile of up to 16384 scores staged in LDS: thread t of a THREADS-thread
// workgroup owns entries t*ITEMS .. t*ITEMS+ITEMS-1, stored with 4 pad words
// after every ITEMS entries so that the owners' 16-byte reads of their own
// entries hit distinct bank groups.
template <int THREADS, int ITEMS>
struct Tile {
  static constexpr int kPitch = ITEMS + 4;
  static constexpr int kFloats = THREADS * kPitch;
  static __device__ __forceinline__ int pos(int e) { return e + 4 * (e / ITEMS); }

  // Issue the coalesced 16-byte loads of scores [0, n) (entries at and past
  // n are NaN); store() then puts them into LDS.
  struct Loads {
    f32x4 v[ITEMS / 4];
  };
  static __device__ __forceinline__ Loads load(const float* src, int n) {
    Loads r;
    const int tid = threadIdx.x;
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
#pragma unroll
    for (int q = 0; q < ITEMS / 4; ++q) {
      const int e = 4 * (q * THREADS + tid);
      if (vec && e + 4 <= n) {
        r.v[q] = *reinterpret_cast<const f32x4*>(src + e);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float t = src[e + u < n ? e + u : 0];
          r.v[q][u] = e + u < n ? t : __builtin_nanf("");
        }
      }
    }
    return r;
  }
  // Store the loads, barrier, and read this thread's own entries into x.
  static __device__ __forceinline__ void store(const Loads& r, float* stage, float (&x)[ITEMS]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < ITEMS / 4; ++q) *reinterpret_cast<f32x4*>(stage + pos(4 * (q * THREADS + tid))) = r.v[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < ITEMS / 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + tid * kPitch + 4 * q);
#pragma unroll
      for (int u = 0; u < 4; ++u) x[4 * q + u] = v[u];
    }
  }
};
using PartTile = Tile<kThreads, kItems>;

struct Shared {
  Filt::Shared fs;
  int32_t si[kStage + 64];  // staged output: entry and score (64 lane-private dump slots at the end)
  float sv[kStage + 64];
  alignas(16) float stage[PartTile::kFloats];
};

// The merge: 512 threads, 32 candidate slots each (1024 x 16 measured slower:
// more waves per barrier, no less latency per phase).
constexpr int kMThreads = 512;
constexpr int kMItems = 32;
static_assert(kMThreads * kMItems == kPart, "merge tile");
using MergeTile = Tile<kMThreads, kMItems>;
using MFilt = sel::Filter<kMThreads, kMItems, 16>;
struct MShared {
  MFilt::Shared fs;
  int32_t si[kStage + 64];  // 64 lane-private dump slots at the end
  float sv[kStage + 64];
  alignas(16) float stage[MergeTile::kFloats];
  int wtot[kMThreads / 64];
};

__device__ __forceinline__ int64_t row_visible(const TopkArgs& a, int64_t row) {
  SeqLayout l;
  l.lens = a.lens;
  const int64_t tpos = seq_len(l, a.n_ctx, a.T, row / a.T) - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  return nv < 0 ? 0 : nv;
}


// Stage 1: per-part local selection.
__global__ __launch_bounds__(kThreads) void topk_part_kernel(TopkArgs a, int64_t nparts, int64_t cap,
                                                             float* cval, int32_t* cidx, int32_t* ccnt) {
  __shared__ Shared sh;
  const int64_t lrow = blockIdx.x / nparts;
  const int64_t part = blockIdx.x % nparts;
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
  float v[kItems];
  PartTile::store(PartTile::load(s, static_cast<int>(cnt)), sh.stage, v);
  const int i0 = tid * kItems;  // this thread's entries i0 .. i0+31 of the part
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

// Merge from the compact lists when they are enough.  Every part's list
// holds all its candidates >= V_p (its smallest listed score, at most its
// lrank-th largest); U is their union, in index order.  With theta_U the k-th largest
// of U (a subset of the row, so theta_U <= the row's k-th largest theta), an
// entry of the row's top-k has a score >= theta >= theta_U; when every V_p <=
// theta_U that score is >= its part's V_p, so the entry is in U and the
// top-k of U is the row's.  Returns false (nothing written) when a list is
// missing or too long, U has fewer than k entries, or some V_p > theta_U.
constexpr int kUItems = kMergeUnion / kMThreads;  // 8
using USel = sel::Select<kMThreads, kUItems>;
static_assert(sizeof(float) * kMergeUnion * 2 <= sizeof(float) * MergeTile::kFloats, "the union fits the stage");

__device__ __forceinline__ bool merge_compact(const TopkArgs& a, int64_t lrow, int nparts, const IndexCandidates& c,
                                              MShared& sh, int32_t* o, float* os) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // The staging below gives each list kMThreads / nparts threads of
  // kMergeUnion / kMThreads entries each.
  if (c.lcap > static_cast<int64_t>(kMergeUnion / kMThreads) * (kMThreads / nparts)) return false;
  const int64_t unit0 = lrow * nparts;
  const int lc = tid < nparts ? c.lcnt[unit0 + tid] : 0;
  const float lt = tid < nparts ? c.lthr[unit0 + tid] : -INFINITY;
  // per wave: any missing list, the lists' total, the largest V_p
  const uint32_t neg = static_cast<uint32_t>(__popcll(__ballot(lc < 0)));
  const uint32_t cnt = static_cast<uint32_t>(lc > 0 ? lc : 0);
  const uint32_t incl = wave_incl_scan(cnt);
  const float vmax_w = wave_max(lt);
  uint32_t* uoff = reinterpret_cast<uint32_t*>(sh.si);  // list offsets in U (<= 256 parts)
  if (sel::lane_id() == 63) {
    sh.fs.wsum[wave] = incl;
    sh.fs.red[0][wave] = vmax_w;
    sh.fs.core.red[0][wave] = neg;
  }
  __syncthreads();
  uint32_t before = 0, total = 0, nneg = 0;
  float vmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMThreads / 64; ++w) {
    before += w < wave ? sh.fs.wsum[w] : 0u;
    total += sh.fs.wsum[w];
    nneg += sh.fs.core.red[0][w];
    vmax = fmaxf(vmax, sh.fs.red[0][w]);
  }
  if (nneg != 0 || total < static_cast<uint32_t>(a.k) || total > static_cast<uint32_t>(kMergeUnion)) {
    __syncthreads();  // the LDS read above is done before the full merge reuses it
    return false;
  }
  if (tid < nparts) uoff[tid] = before + incl - cnt;
  __syncthreads();
  // U into LDS (values, then indices): kMThreads / nparts threads per list,
  // all loads issued before any store (one memory round trip).
  float* uval = sh.stage;
  int32_t* uidx = reinterpret_cast<int32_t*>(sh.stage + kMergeUnion);
  {
    constexpr int kR = kMergeUnion / kMThreads;  // entries per thread: lcap * nparts <= kMergeUnion
    const int tpp = kMThreads / nparts;          // >= 2 (nparts <= 256)
    const int p = tid / tpp, li = tid % tpp;
    const int n = p < nparts ? c.lcnt[unit0 + p] : 0;
    const float* lvp = c.lval + (unit0 + (p < nparts ? p : 0)) * c.lcap;
    const int32_t* lip = c.lidx + (unit0 + (p < nparts ? p : 0)) * c.lcap;
    float tv[kR];
    int32_t tx[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int i = li + r * tpp;
      const int ic = i < n ? i : 0;  // in range: lcap >= 1
      tv[r] = lvp[ic];
      tx[r] = lip[ic];
    }
    const uint32_t off = p < nparts ? uoff[p] : 0u;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int i = li + r * tpp;
      if (i < n) {
        uval[off + i] = tv[r];
        uidx[off + i] = tx[r];
      }
    }
  }
  USel::zero(sh.fs.core);
  __syncthreads();
  uint32_t keys[kUItems];
  uint32_t vm = 0;
#pragma unroll
  for (int j = 0; j < kUItems; ++j) {
    const uint32_t u = static_cast<uint32_t>(tid * kUItems + j);
    keys[j] = float_key(uval[u < total ? u : 0]);
    vm |= static_cast<uint32_t>(u < total) << j;
  }
  uint32_t thr, take;
  USel::radix_select(keys, vm, static_cast<uint32_t>(a.k), sh.fs.core, &thr, &take);
  if (vmax > key_float(thr)) {  // uniform: some part's list may miss row top-k entries
    __syncthreads();
    return false;
  }
  uint32_t bg = 0, be = 0;
  USel::compact(keys, vm, thr, take, sh.fs.core, &bg, &be, [&](int j, uint32_t pos) {
    const int u = tid * kUItems + j;
    sh.sv[pos] = uval[u];
    sh.si[pos + kStage / 2] = uidx[u];  // past the list offsets
  });
  for (int i = tid; i < a.k; i += kMThreads) {
    o[i] = sh.si[i + kStage / 2];
    if (os) os[i] = sh.sv[i];
  }
  return true;
}

// Fast merge: nparts * cap <= 16384 slots and nparts <= 256.  The candidate
// values are staged in LDS with coalesced loads and thread t holds slots
// 32t .. 32t+31; slots without a candidate hold NaN.
__global__ __launch_bounds__(kMThreads) void topk_merge_kernel(TopkArgs a, int nparts, IndexCandidates c,
                                                               bool fused) {
  __shared__ MShared sh;
  const int64_t lrow = blockIdx.x;
  if (!fused && merge_trivial(a, lrow)) return;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;
  const int cap = static_cast<int>(c.cap);
  const int ns = nparts * cap;
  const float* rv = c.cval + lrow * ns;
  const int32_t* ri = c.cidx + lrow * ns;
  const int32_t* rc = c.ccnt + lrow * nparts;
  if (c.lval && merge_compact(a, lrow, nparts, c, sh, o, os)) return;
  // Candidate slots past their part's count hold NaN (written so by the part
  // stage), as does everything past the last part: no validity test here.
  // The candidate loads go out first; the part counts are summed meanwhile.
  const MergeTile::Loads ld = MergeTile::load(rv, ns);
  MFilt::zero(sh.fs);
  static_assert(kMaxMergeParts <= kMThreads, "one part count per thread");
  const int pc = static_cast<int>(sel::wave_sum(static_cast<uint32_t>(tid < nparts ? rc[tid] : 0)));
  if (lane_id() == 0) sh.wtot[tid >> 6] = pc;
  float v[kMItems];
  MergeTile::store(ld, sh.stage, v);  // its barrier also publishes wtot
  int total = 0;  // valid candidates of the row
#pragma unroll
  for (int w = 0; w < kMThreads / 64; ++w) total += sh.wtot[w];
  const int s0 = tid * kMItems;
  if (total <= a.k) {  // every valid candidate is kept, in slot order; -1 padding after them
    for (int64_t i = total + tid; i < a.k; i += kMThreads) {
      o[i] = -1;
      if (os) os[i] = -INFINITY;
    }
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kMItems; ++j) c += v[j] == v[j];
    const uint32_t incl = wave_incl_scan(c);
    if (lane_id() == 63) sh.fs.core.wsum[tid >> 6] = incl;
    __syncthreads();
    uint32_t pos = incl - c;
    for (int w = 0; w < (tid >> 6); ++w) pos += sh.fs.core.wsum[w];
#pragma unroll
    for (int j = 0; j < kMItems; ++j)
      if (v[j] == v[j]) {
        o[pos] = ri[s0 + j];
        if (os) os[pos] = v[j];
        ++pos;
      }
    return;
  }
  const uint32_t uk = static_cast<uint32_t>(a.k);
  float vmin, vmax;
  MFilt::block_range(v, sh.fs, &vmin, &vmax);
  auto src = [&](uint32_t e) { return sh.stage[MergeTile::pos(static_cast<int>(e))]; };
  if (a.k <= kStage) {  // stage the kept candidates in LDS, then store coalesced
    MFilt::run(
        v, src, static_cast<uint32_t>(total), uk, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t e) {
          const uint32_t p = pos != sel::kNoSlot ? pos : kStage + lane_id();
          sh.si[p] = static_cast<int32_t>(e);
          sh.sv[p] = val;
        },
        [&](int j, uint32_t pos) {
          sh.si[pos] = s0 + j;
          sh.sv[pos] = sh.stage[MergeTile::pos(s0 + j)];
        });
    for (int i = tid; i < a.k; i += kMThreads) {
      o[i] = ri[sh.si[i]];
      if (os) os[i] = sh.sv[i];
    }
  } else {
    MFilt::run(
        v, src, static_cast<uint32_t>(total), uk, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t e) {
          if (pos == sel::kNoSlot) return;
          o[pos] = ri[e];
          if (os) os[pos] = val;
        },
        [&](int j, uint32_t pos) {
          o[pos] = ri[s0 + j];
          if (os) os[pos] = sh.stage[MergeTile::pos(s0 + j)];
        });
  }
}

// General merge (k >= 16384, or more than 256 parts): histogram passes over
// the slots in L2, then ordered compaction tile by tile.
__global__ __launch_bounds__(kThreads) void topk_merge_general(TopkArgs a, int64_t nparts, int64_t cap,
                                                               const float* cval, const int32_t* cidx,
                                                               const int32_t* ccnt) {
  __shared__ struct { Sel::Shared core; } sh;
  const int64_t lrow = blockIdx.x;
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

int64_t topk_parts(int64_t L) { return L <= 0 ? 1 : (L + kPart - 1) / kPart; }
int64_t topk_cap(int64_t k) { return k < kPart ? k : kPart; }

size_t topk_ws_bytes_per_row(int64_t L, int64_t k) {
  const int64_t np = topk_parts(L);
  const size_t b = static_cast<size_t>(np) * topk_cap(k) * 8 + static_cast<size_t>(np) * 4;
  return (b + 255) / 256 * 256;
}

hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t s) {
  if (a.nrows == 0 || a.k == 0) return hipSuccess;
  const int64_t np = topk_parts(a.L), cap = topk_cap(a.k);
  float* cval = static_cast<float*>(ws);
  int32_t* cidx = reinterpret_cast<int32_t*>(cval + a.nrows * np * cap);
  int32_t* ccnt = cidx + a.nrows * np * cap;
  hipLaunchKernelGGL(topk_part_kernel, dim3(static_cast<uint32_t>(a.nrows * np)), dim3(kThreads), 0, s, a, np,
                     cap, cval, cidx, ccnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  IndexCandidates c;
  c.cval = cval;
  c.cidx = cidx;
  c.ccnt = ccnt;
  c.cap = cap;
  return launch_topk_merge(a, np, c, false, s);
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
