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

namespace csa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 32;
constexpr int64_t kPart = static_cast<int64_t>(kThreads) * kItems;  // 16384
constexpr int kBins = 2048;
constexpr int kMaxMergeParts = 256;  // part counts cached in LDS by the merge
constexpr int kStage = 2048;         // outputs up to this size are staged in LDS, then stored coalesced
constexpr int kSmall = 256;          // a threshold bin with at most this many keys is resolved by one wave

struct Shared {
  uint32_t hist[2][kBins];
  uint32_t red[2][2 * kWaves];
  uint32_t wsum[kWaves];
  uint32_t sel_bin, sel_above;
  int32_t pcnt[kMaxMergeParts];
  int32_t si[kStage];
  uint32_t ck[kSmall];  // keys of the threshold bin
  uint32_t ncand, thr, take;
};

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, 64);
    if (static_cast<int>(lane_id()) >= o) v += y;
  }
  return v;
}

// One histogram pass over the keys selected by `inb` (per-thread item mask):
// bins from bin(j) (in 0 .. nb-1, ascending with the key), then the bin that
// holds the remaining-th largest.  Returns that bin and subtracts the count of
// keys in higher bins from *remaining.  Expects sh.hist[buf] zeroed and a
// barrier since; zeroes sh.hist[buf ^ 1] for the next pass.
template <typename BinOf>
__device__ __forceinline__ uint32_t hist_pass(uint32_t inb, int nb, BinOf bin_of, Shared& sh, int buf,
                                              uint32_t* remaining) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  constexpr int kBpt = kBins / kThreads;  // bins per thread in the scan
  uint32_t* h = sh.hist[buf];
#pragma unroll
  for (int j = 0; j < kItems; ++j)
    if ((inb >> j) & 1u) atomicAdd(&h[bin_of(j)], 1u);
  uint32_t* hn = sh.hist[buf ^ 1];
#pragma unroll
  for (int i = 0; i < kBpt; ++i) hn[tid + i * kThreads] = 0;
  __syncthreads();
  // Bins from the top: thread t owns bins nb-1-kBpt*t .. nb-kBpt*(t+1).
  uint32_t c[kBpt], s = 0;
#pragma unroll
  for (int q = 0; q < kBpt; ++q) {
    const int bq = nb - 1 - kBpt * tid - q;
    c[q] = bq >= 0 ? h[bq] : 0u;
    s += c[q];
  }
  const uint32_t incl = wave_incl_scan(s);
  if (lane_id() == 63) sh.wsum[wave] = incl;
  __syncthreads();
  uint32_t excl = incl - s;
  for (int w = 0; w < wave; ++w) excl += sh.wsum[w];
  const uint32_t rem = *remaining;
#pragma unroll
  for (int q = 0; q < kBpt; ++q) {
    const int bq = nb - 1 - kBpt * tid - q;
    if (bq >= 0 && excl < rem && excl + c[q] >= rem) {
      sh.sel_bin = static_cast<uint32_t>(bq);
      sh.sel_above = excl;
    }
    excl += c[q];
  }
  __syncthreads();
  *remaining = rem - sh.sel_above;
  return sh.sel_bin;
}

// Min and max of the keys selected by `inb` over the workgroup.
__device__ __forceinline__ void block_minmax(const uint32_t (&keys)[kItems], uint32_t inb, Shared& sh, int slot,
                                             uint32_t* kmin_out, uint32_t* kmax_out) {
  const int wave = threadIdx.x >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kItems; ++j)
    if ((inb >> j) & 1u) {
      kmin = keys[j] < kmin ? keys[j] : kmin;
      kmax = keys[j] > kmax ? keys[j] : kmax;
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t a = __shfl_xor(kmin, o, 64), b = __shfl_xor(kmax, o, 64);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  if (lane_id() == 0) {
    sh.red[slot][2 * wave] = kmin;
    sh.red[slot][2 * wave + 1] = kmax;
  }
  __syncthreads();
  kmin = sh.red[slot][0];
  kmax = sh.red[slot][1];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    kmin = sh.red[slot][2 * w] < kmin ? sh.red[slot][2 * w] : kmin;
    kmax = sh.red[slot][2 * w + 1] > kmax ? sh.red[slot][2 * w + 1] : kmax;
  }
  *kmin_out = kmin;
  *kmax_out = kmax;
}

// Radix select over the valid keys held by the workgroup (keys[j] valid iff
// bit j of vmask).  Finds the key of the sel-th largest (1-based, sel <= number
// of valid keys) and how many keys equal to it are kept (the lowest-indexed).
// Expects sh.hist[0] and sh.ncand zeroed and a barrier since.
//
// First pass: 2048 bins linear in the score between the extremes (a
// monotone map, so bins are ordered like the keys and equal scores share a
// bin).  Indexer scores are bell-shaped, so this spreads them thinly where
// bins of the key bits would pile a part onto a handful of bins (LDS atomics
// to one bin serialise).  The keys of the chosen bin are then resolved by
// passes of up to 11 key bits below their common bit prefix.  Non-finite
// extremes fall back to key-bit passes throughout.
__device__ __forceinline__ void radix_select(const uint32_t (&keys)[kItems], uint32_t vmask, uint32_t sel,
                                             Shared& sh, uint32_t* thr_out, uint32_t* take_eq_out) {
  uint32_t kmin, kmax;
  block_minmax(keys, vmask, sh, 0, &kmin, &kmax);
  uint32_t remaining = sel;
  uint32_t inb = vmask;  // keys still in the running
  int buf = 0;
  const float vmin = key_float(kmin), vmax = key_float(kmax);
  const float range = vmax - vmin;
  const float scale = static_cast<float>(kBins) / range;
  if (kmin != kmax && __builtin_isfinite(vmin) && __builtin_isfinite(vmax) && __builtin_isfinite(range) &&
      range > 0.f && __builtin_isfinite(scale)) {
    auto vbin = [&](int j) {
      const float x = (key_float(keys[j]) - vmin) * scale;
      const int bb = static_cast<int>(x);
      return bb < kBins - 1 ? bb : kBins - 1;
    };
    const uint32_t b = hist_pass(inb, kBins, vbin, sh, buf, &remaining);
    buf ^= 1;
    // The threshold lies among the keys of bin b (typically a few dozen):
    // gather them and let one wavefront find the remaining-th largest by
    // counting, instead of more passes over every item.
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const bool in = ((inb >> j) & 1u) && vbin(j) == static_cast<int>(b);
      m |= static_cast<uint32_t>(in) << j;
      if (in) {
        const uint32_t slot = atomicAdd(&sh.ncand, 1u);
        if (slot < kSmall) sh.ck[slot] = keys[j];
      }
    }
    inb &= m;
    __syncthreads();
    const uint32_t n = sh.ncand;
    if (n <= kSmall) {
      if ((threadIdx.x >> 6) == 0) {
        const uint32_t lane = lane_id();
        uint32_t mk[kSmall / 64], gt[kSmall / 64], ge[kSmall / 64];
#pragma unroll
        for (int q = 0; q < kSmall / 64; ++q) {
          mk[q] = lane + 64 * q < n ? sh.ck[lane + 64 * q] : 0u;
          gt[q] = 0;
          ge[q] = 0;
        }
        for (uint32_t i = 0; i < n; ++i) {
          const uint32_t x = sh.ck[i];
#pragma unroll
          for (int q = 0; q < kSmall / 64; ++q) {
            gt[q] += x > mk[q];
            ge[q] += x >= mk[q];
          }
        }
#pragma unroll
        for (int q = 0; q < kSmall / 64; ++q)
          if (lane + 64 * q < n && gt[q] < remaining && ge[q] >= remaining) {
            sh.thr = mk[q];
            sh.take = remaining - gt[q];
          }
      }
      __syncthreads();
      *thr_out = sh.thr;
      *take_eq_out = sh.take;
      return;
    }
    block_minmax(keys, inb, sh, 1, &kmin, &kmax);
  }
  const uint32_t diff = kmin ^ kmax;
  uint32_t prefix = diff ? (kmax & ~((2u << (31 - __clz(diff))) - 1u)) : kmax;
  int top = diff ? 31 - __clz(diff) : -1;  // highest undecided bit
  while (top >= 0) {
    const int width = top + 1 < 11 ? top + 1 : 11;
    const int shift = top + 1 - width;
    const int nb = 1 << width;
    const uint32_t hi_mask = ~((2u << top) - 1u);  // decided bits (all of them when top = 31 ... 0)
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) m |= static_cast<uint32_t>((keys[j] & hi_mask) == (prefix & hi_mask)) << j;
    inb &= m;
    const uint32_t b =
        hist_pass(inb, nb, [&](int j) { return static_cast<int>((keys[j] >> shift) & (nb - 1)); }, sh, buf,
                  &remaining);
    buf ^= 1;
    prefix = (prefix & hi_mask) | (b << shift);
    top = shift - 1;
  }
  *thr_out = prefix;
  *take_eq_out = remaining;
}

// Ordered compaction of one tile (item j of thread t = tile entry t*32 + j,
// valid iff bit j of vmask): kept items (key > thr, or key == thr among the
// first take_eq such items of the whole sequence of tiles) get consecutive
// output slots in entry order after *base_gt / *base_eq earlier ones.  A tile
// holds at most 16384 entries, so both counts fit 16-bit halves of one scan.
// emit(j, slot) runs only for kept items (a few per thread): the thread's kept
// mask is built first and its set bits are walked.
template <typename Emit>
__device__ __forceinline__ void compact_tile(const uint32_t (&keys)[kItems], uint32_t vmask, uint32_t thr,
                                             uint32_t take_eq, Shared& sh, uint32_t* base_gt, uint32_t* base_eq,
                                             Emit emit) {
  const int wave = threadIdx.x >> 6;
  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    gtm |= static_cast<uint32_t>(keys[j] > thr) << j;
    eqm |= static_cast<uint32_t>(keys[j] == thr) << j;
  }
  gtm &= vmask;
  eqm &= vmask;
  const uint32_t neq = __popc(eqm);
  const uint32_t packed = (neq << 16) | static_cast<uint32_t>(__popc(gtm));
  const uint32_t incl = wave_incl_scan(packed);
  if (lane_id() == 63) sh.wsum[wave] = incl;
  __syncthreads();
  uint32_t excl = incl - packed, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    excl += w < wave ? sh.wsum[w] : 0u;
    total += sh.wsum[w];
  }
  const uint32_t gt0 = *base_gt + (excl & 0xffffu);  // greater items before this thread
  const uint32_t eq0 = *base_eq + (excl >> 16);      // equal items before this thread
  // This thread keeps its lowest min(neq, take_eq - eq0) equal items.
  uint32_t keq = take_eq > eq0 ? take_eq - eq0 : 0u;
  uint32_t em = eqm, km = gtm;
  while (keq > 0 && em) {
    const uint32_t bit = em & (0u - em);
    km |= bit;
    em ^= bit;
    --keq;
  }
  uint32_t slot = gt0 + (eq0 < take_eq ? eq0 : take_eq);  // kept items before this thread
  while (km) {
    const int j = __builtin_ctz(km);
    km &= km - 1u;
    emit(j, slot++);
  }
  *base_gt += total & 0xffffu;
  *base_eq += total >> 16;
  __syncthreads();  // wsum is reused by the next scan
}

__device__ __forceinline__ int64_t row_visible(const TopkArgs& a, int64_t row) {
  const int64_t tpos = a.n_ctx - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  return nv < 0 ? 0 : nv;
}

__device__ __forceinline__ void zero_hist0(Shared& sh) {
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[0][i] = 0;
  if (threadIdx.x == 0) sh.ncand = 0;
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
  if (cnt <= 0) {
    if (threadIdx.x == 0) *cc = 0;
    return;
  }
  zero_hist0(sh);
  const float* s = a.score + lrow * a.ld + base;
  float* ov = cval + (lrow * nparts + part) * cap;
  int32_t* oi = cidx + (lrow * nparts + part) * cap;
  const int tid = threadIdx.x;
  const int i0 = tid * kItems;  // this thread's entries i0 .. i0+31 of the part
  float v[kItems];
  uint32_t keys[kItems];
  const int nvalid = cnt - i0 <= 0 ? 0 : (cnt - i0 >= kItems ? kItems : static_cast<int>(cnt - i0));
  const uint32_t vmask = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
  if (nvalid == kItems && (reinterpret_cast<uintptr_t>(s) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(s + i0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j) v[j] = s[j < nvalid ? i0 + j : 0];
  }
#pragma unroll
  for (int j = 0; j < kItems; ++j) keys[j] = float_key(v[j]);
  if (cnt <= cap) {  // the whole part is kept
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (j < nvalid) {
        ov[i0 + j] = v[j];
        oi[i0 + j] = static_cast<int32_t>(base + i0 + j);
      }
    if (tid == 0) *cc = static_cast<int32_t>(cnt);
    return;
  }
  __syncthreads();
  uint32_t thr, take_eq;
  radix_select(keys, vmask, static_cast<uint32_t>(cap), sh, &thr, &take_eq);
  uint32_t bg = 0, be = 0;
  if (cap <= kStage) {  // stage the kept entries in LDS, then store them coalesced
    compact_tile(keys, vmask, thr, take_eq, sh, &bg, &be,
                 [&](int j, uint32_t pos) { sh.si[pos] = i0 + j; });
    for (int i = tid; i < cap; i += kThreads) {
      const int li = sh.si[i];
      ov[i] = s[li];
      oi[i] = static_cast<int32_t>(base + li);
    }
  } else {
    compact_tile(keys, vmask, thr, take_eq, sh, &bg, &be, [&](int j, uint32_t pos) {
      ov[pos] = s[i0 + j];
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
  for (int64_t i = threadIdx.x; i < a.k; i += kThreads) {
    o[i] = i < nv ? static_cast<int32_t>(i) : -1;
    if (os) os[i] = i < nv ? s[i] : -INFINITY;
  }
  return true;
}

// Fast merge: nparts * cap <= 16384 slots and nparts <= 256.  Thread t holds
// slots 32t .. 32t+31; part counts come from LDS, and the part of a slot is an
// exact multiply-high (slot * cap < 2^32 here).
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(TopkArgs a, int nparts, int cap, const float* cval,
                                                              const int32_t* cidx, const int32_t* ccnt) {
  __shared__ Shared sh;
  const int64_t lrow = blockIdx.x;
  if (merge_trivial(a, lrow)) return;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;
  const int ns = nparts * cap;
  const float* rv = cval + lrow * ns;
  const int32_t* ri = cidx + lrow * ns;
  const int32_t* rc = ccnt + lrow * nparts;
  zero_hist0(sh);
  for (int p = tid; p < nparts; p += kThreads) sh.pcnt[p] = rc[p];
  __syncthreads();
  const uint32_t ucap = static_cast<uint32_t>(cap);
  const uint32_t magic = static_cast<uint32_t>((0x100000000ull + ucap - 1) / ucap);
  uint32_t keys[kItems];
  float v[kItems];
  int32_t ix[kItems];
  const int s0 = tid * kItems;
  if (s0 + kItems <= ns && ((reinterpret_cast<uintptr_t>(rv + s0) | reinterpret_cast<uintptr_t>(ri + s0)) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(rv + s0 + 4 * q);
      const u32x4 y = *reinterpret_cast<const u32x4*>(ri + s0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[4 * q + e] = x[e];
        ix[4 * q + e] = static_cast<int32_t>(y[e]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int sc = s0 + j < ns ? s0 + j : ns - 1;
      v[j] = rv[sc];
      ix[j] = ri[sc];
    }
  }
  uint32_t vmask = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int sl = s0 + j;
    const int sc = sl < ns ? sl : ns - 1;
    const uint32_t pp = __umulhi(static_cast<uint32_t>(sc), magic);
    const bool ok = sl < ns && static_cast<int>(static_cast<uint32_t>(sc) - pp * ucap) < sh.pcnt[pp];
    vmask |= static_cast<uint32_t>(ok) << j;
    keys[j] = float_key(v[j]);
  }
  uint32_t thr, take_eq;
  radix_select(keys, vmask, static_cast<uint32_t>(a.k), sh, &thr, &take_eq);
  uint32_t bg = 0, be = 0;
  if (a.k <= kStage) {  // stage the kept slots in LDS, then store coalesced
    compact_tile(keys, vmask, thr, take_eq, sh, &bg, &be,
                 [&](int j, uint32_t pos) { sh.si[pos] = s0 + j; });
    for (int i = tid; i < a.k; i += kThreads) {
      const int sl = sh.si[i];
      o[i] = ri[sl];
      if (os) os[i] = rv[sl];
    }
  } else {
    compact_tile(keys, vmask, thr, take_eq, sh, &bg, &be, [&](int j, uint32_t pos) {
      o[pos] = ri[s0 + j];
      if (os) os[pos] = rv[s0 + j];
    });
  }
}

// General merge (k >= 16384, or more than 256 parts): histogram passes over
// the slots in L2, then ordered compaction tile by tile.
__global__ __launch_bounds__(kThreads) void topk_merge_general(TopkArgs a, int64_t nparts, int64_t cap,
                                                               const float* cval, const int32_t* cidx,
                                                               const int32_t* ccnt) {
  __shared__ Shared sh;
  const int64_t lrow = blockIdx.x;
  if (merge_trivial(a, lrow)) return;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;
  const int64_t nslots = nparts * cap;
  const float* rv = cval + lrow * nparts * cap;
  const int32_t* ri = cidx + lrow * nparts * cap;
  const int32_t* rc = ccnt + lrow * nparts;
  zero_hist0(sh);
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
    uint32_t* h = sh.hist[pass & 1];
    for (int64_t sl = tid; sl < nslots; sl += kThreads) {
      if (!slot_ok(sl)) continue;
      const uint32_t key = float_key(rv[sl]);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1u);
    }
    for (int i = tid; i < kBins; i += kThreads) sh.hist[(pass & 1) ^ 1][i] = 0;
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
    if (lane_id() == 63) sh.wsum[tid >> 6] = incl;
    __syncthreads();
    uint32_t excl = incl - s;
    for (int w = 0; w < (tid >> 6); ++w) excl += sh.wsum[w];
#pragma unroll
    for (int q = 0; q < kBpt; ++q) {
      const int bq = nb - 1 - kBpt * tid - q;
      if (bq >= 0 && excl < remaining && excl + c[q] >= remaining) {
        sh.sel_bin = static_cast<uint32_t>(bq);
        sh.sel_above = excl;
      }
      excl += c[q];
    }
    __syncthreads();
    prefix |= sh.sel_bin << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    remaining -= sh.sel_above;
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
    compact_tile(keys, vmask, prefix, remaining, sh, &bg, &be, [&](int j, uint32_t pos) {
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
  if (np * cap <= kPart && np <= kMaxMergeParts)
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a,
                       static_cast<int>(np), static_cast<int>(cap), cval, cidx, ccnt);
  else
    hipLaunchKernelGGL(topk_merge_general, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a, np, cap,
                       cval, cidx, ccnt);
  return hipGetLastError();
}

}  // namespace csa
