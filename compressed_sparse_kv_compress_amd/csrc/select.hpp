// Workgroup-wide exact top-k selection over keys held in registers, shared by
// the top-k kernels and by the indexer's fused part selection.
//
// Keys are order-preserving uint32 images of fp32 scores (-0 and +0 equal).
// THREADS threads hold ITEMS keys each; item j of thread t is entry
// t * ITEMS + j of the tile, and the valid ones are flagged in a per-thread
// bit mask.  radix_select finds the key of the sel-th largest valid key and
// how many keys equal to it are kept (the lowest-indexed ones); compact gives
// every kept item its output slot in entry order.
//
// Selection (all passes are latency / issue bound at these sizes, so the
// number of passes over all items is what is minimised):
//   1. min / max reduction;
//   2. one histogram pass over 2048 bins linear in the score between min and
//      max: a monotone map, so bins are ordered like the keys and equal scores
//      share a bin, and bell-shaped scores spread thinly (bins of the keys'
//      top bits pile them onto a handful of bins, whose LDS atomics serialise);
//   3. the keys of the threshold bin (typically a few dozen) are gathered in
//      LDS and one wavefront finds the remaining-th largest by counting; more
//      than kSmall such keys (ties, odd distributions) or non-finite extremes
//      fall back to passes of up to 11 key bits below their common prefix.
// Compaction: one 32-bit workgroup scan of per-thread (greater, equal) counts
// packed in 16-bit halves (a tile holds at most 65535 entries), then every
// thread walks only its kept items.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace csa {
namespace sel {

constexpr int kBins = 2048;
constexpr int kSmall = 256;  // a threshold bin with at most this many keys is resolved by one wavefront
constexpr uint32_t kNoSlot = 0xffffffffu;  // emit position of a survivor that is not kept

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<kRowShr1>(0u, v);
  v += dpp<kRowShr2>(0u, v);
  v += dpp<kRowShr4>(0u, v);
  v += dpp<kRowShr8>(0u, v);
  v += dpp<kRowBcast15, 0xa>(0u, v);
  v += dpp<kRowBcast31, 0xc>(0u, v);
  return v;
}

// Wave-uniform max / min / sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = f(v, dpp<kRowShr1>(0u, v));
  v = f(v, dpp<kRowShr2>(0u, v));
  v = f(v, dpp<kRowShr4>(0u, v));
  v = f(v, dpp<kRowShr8>(0u, v));
  v = f(v, dpp<kRowBcast15, 0xa>(0u, v));
  v = f(v, dpp<kRowBcast31, 0xc>(0u, v));
  return last_lane(v);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  constexpr uint32_t id = 0xffffffffu;
  v = f(v, dpp<kRowShr1>(id, v));
  v = f(v, dpp<kRowShr2>(id, v));
  v = f(v, dpp<kRowShr4>(id, v));
  v = f(v, dpp<kRowShr8>(id, v));
  v = f(v, dpp<kRowBcast15, 0xa>(id, v));
  v = f(v, dpp<kRowBcast31, 0xc>(id, v));
  return last_lane(v);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return last_lane(wave_incl_scan(v)); }

// LDS of a selection by a THREADS-thread workgroup (any items per thread).
template <int THREADS>
struct SelectShared {
  uint32_t hist[2][kBins];
  uint32_t red[2][2 * (THREADS / 64)];
  uint32_t wsum[THREADS / 64];
  uint32_t sel_bin, sel_above;
  uint32_t ck[kSmall + 64];  // keys of the threshold bin; 64 lane-private dump slots after them
  uint32_t ncand, thr, take;
};

// Stores the items flagged in m (bit j: item j) at dst[pos], dst[pos+1], ...
// in item order, branch-free: unflagged items (and flagged ones at or past
// limit) go to dst[dump].
template <int N, typename M, typename T, typename Val>
__device__ __forceinline__ void scatter_flagged(M m, uint32_t pos, uint32_t limit, uint32_t dump, T* dst, Val val) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const bool in = (m >> j) & 1u;
    dst[in && pos < limit ? pos : dump] = val(j);
    pos += in;
  }
}

template <int THREADS, int ITEMS>
struct Select {
  static_assert(THREADS % 64 == 0 && kBins % THREADS == 0, "workgroup shape");
  static_assert(ITEMS <= 64 && THREADS * ITEMS < 65536, "packed 16-bit compaction counts");
  static constexpr int kWaves = THREADS / 64;
  static constexpr int kBpt = kBins / THREADS;  // bins per thread in the scan
  using Mask = std::conditional_t<(ITEMS > 32), uint64_t, uint32_t>;
  using Shared = SelectShared<THREADS>;

  static __device__ __forceinline__ uint32_t popc(Mask m) {
    if constexpr (sizeof(Mask) == 8) return static_cast<uint32_t>(__popcll(m));
    else return static_cast<uint32_t>(__popc(m));
  }
  static __device__ __forceinline__ int ctz(Mask m) {
    if constexpr (sizeof(Mask) == 8) return __builtin_ctzll(m);
    else return __builtin_ctz(m);
  }
  static __device__ __forceinline__ bool bit(Mask m, int j) { return (m >> j) & 1u; }

  // Zero what radix_select expects zeroed (hist[0], the gather count); a
  // barrier must follow before radix_select.
  static __device__ __forceinline__ void zero(Shared& sh) {
    for (int i = threadIdx.x; i < kBins; i += THREADS) sh.hist[0][i] = 0;
    if (threadIdx.x == 0) sh.ncand = 0;
  }

  // One histogram pass over the keys selected by `inb`: bins from bin_of(j)
  // (0 .. nb-1, ascending with the key), then the bin that holds the
  // remaining-th largest.  Returns that bin and subtracts the count of keys in
  // higher bins from *remaining.  Expects sh.hist[buf] zeroed and a barrier
  // since; zeroes sh.hist[buf ^ 1] for the next pass.
  template <typename BinOf>
  static __device__ __forceinline__ uint32_t hist_pass(Mask inb, int nb, BinOf bin_of, Shared& sh, int buf,
                                                       uint32_t* remaining) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    uint32_t* h = sh.hist[buf];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (bit(inb, j)) atomicAdd(&h[bin_of(j)], 1u);
    uint32_t* hn = sh.hist[buf ^ 1];
#pragma unroll
    for (int i = 0; i < kBpt; ++i) hn[tid + i * THREADS] = 0;
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

  // Min and max of the keys selected by `inb` over the workgroup (one barrier).
  static __device__ __forceinline__ void block_minmax(const uint32_t (&keys)[ITEMS], Mask inb, Shared& sh, int slot,
                                                      uint32_t* kmin_out, uint32_t* kmax_out) {
    const int wave = threadIdx.x >> 6;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (bit(inb, j)) {
        kmin = keys[j] < kmin ? keys[j] : kmin;
        kmax = keys[j] > kmax ? keys[j] : kmax;
      }
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
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

  // Key of the sel-th largest valid key (1 <= sel <= number of valid keys) and
  // the number of keys equal to it that are kept.  Expects zero(sh) and a
  // barrier since.
  static __device__ __forceinline__ void radix_select(const uint32_t (&keys)[ITEMS], Mask vmask, uint32_t sel,
                                                      Shared& sh, uint32_t* thr_out, uint32_t* take_eq_out) {
    uint32_t kmin, kmax;
    block_minmax(keys, vmask, sh, 0, &kmin, &kmax);
    uint32_t remaining = sel;
    Mask inb = vmask;  // keys still in the running
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
      // The threshold lies among the keys of bin b: gather them (one LDS
      // atomic per wavefront reserves its slots) and let one wavefront find
      // the remaining-th largest by counting.
      Mask m = 0;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) m |= static_cast<Mask>(bit(inb, j) && vbin(j) == static_cast<int>(b)) << j;
      inb &= m;
      const uint32_t c = popc(m);
      const uint32_t incl = wave_incl_scan(c);
      uint32_t base = 0;
      if (lane_id() == 63) base = atomicAdd(&sh.ncand, incl);
      base = last_lane(base);
      if (last_lane(incl) != 0)
        scatter_flagged<ITEMS>(m, base + incl - c, kSmall, kSmall + lane_id(), sh.ck, [&](int j) { return keys[j]; });
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
      const uint32_t hi_mask = ~((2u << top) - 1u);  // decided bits
      Mask m = 0;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) m |= static_cast<Mask>((keys[j] & hi_mask) == (prefix & hi_mask)) << j;
      inb &= m;
      const uint32_t b = hist_pass(
          inb, nb, [&](int j) { return static_cast<int>((keys[j] >> shift) & (nb - 1)); }, sh, buf, &remaining);
      buf ^= 1;
      prefix = (prefix & hi_mask) | (b << shift);
      top = shift - 1;
    }
    *thr_out = prefix;
    *take_eq_out = remaining;
  }

  // Ordered compaction of one tile: kept items (key > thr, or key == thr
  // among the first take_eq such items of the whole sequence of tiles) get
  // consecutive output slots in entry order after *base_gt / *base_eq earlier
  // ones; emit(j, slot) runs only for the kept items of this thread.  Ends
  // with a barrier, so what emit wrote to LDS is visible to the workgroup.
  template <typename Emit>
  static __device__ __forceinline__ void compact(const uint32_t (&keys)[ITEMS], Mask vmask, uint32_t thr,
                                                 uint32_t take_eq, Shared& sh, uint32_t* base_gt, uint32_t* base_eq,
                                                 Emit emit) {
    const int wave = threadIdx.x >> 6;
    Mask gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      gtm |= static_cast<Mask>(keys[j] > thr) << j;
      eqm |= static_cast<Mask>(keys[j] == thr) << j;
    }
    gtm &= vmask;
    eqm &= vmask;
    const uint32_t neq = popc(eqm);
    const uint32_t packed = (neq << 16) | popc(gtm);
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
    Mask em = eqm, km = gtm;
    while (keq > 0 && em) {
      const Mask b = em & (0 - em);
      km |= b;
      em ^= b;
      --keq;
    }
    uint32_t slot = gt0 + (eq0 < take_eq ? eq0 : take_eq);  // kept items before this thread
    while (km) {
      const int j = ctz(km);
      km &= km - 1;
      emit(j, slot++);
    }
    *base_gt += total & 0xffffu;
    *base_eq += total >> 16;
    __syncthreads();  // wsum is reused by the next scan
  }
};

// Float min / max over the 64 lanes of a wavefront, NaN ignored (wave-uniform).
__device__ __forceinline__ float wave_fmin(float v) {
  constexpr uint32_t id = 0x7f800000u;  // +inf
  auto f = [](float a, uint32_t b) { return __builtin_fminf(a, __uint_as_float(b)); };
  v = f(v, dpp<kRowShr1>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowShr2>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowShr4>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowShr8>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowBcast15, 0xa>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowBcast31, 0xc>(id, __float_as_uint(v)));
  return __uint_as_float(last_lane(__float_as_uint(v)));
}
__device__ __forceinline__ float wave_fmax(float v) {
  constexpr uint32_t id = 0xff800000u;  // -inf
  auto f = [](float a, uint32_t b) { return __builtin_fmaxf(a, __uint_as_float(b)); };
  v = f(v, dpp<kRowShr1>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowShr2>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowShr4>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowShr8>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowBcast15, 0xa>(id, __float_as_uint(v)));
  v = f(v, dpp<kRowBcast31, 0xc>(id, __float_as_uint(v)));
  return __uint_as_float(last_lane(__float_as_uint(v)));
}

// Selection through a sampled threshold, in the float domain, for sel well
// below the number of valid scores (a part or a merge tile keeps about one
// score in sixteen).  Thread t holds ITEMS scores, entries t*ITEMS ..
// t*ITEMS+ITEMS-1 of the tile, in registers, and the caller can read entry e
// again from LDS (src(e)); invalid entries are NaN, so every comparison drops
// them and min / max skip them.  Scores are ordered as floats (-0 ties +0);
// the lower entry wins ties.
//   1. a value-linear histogram of kNs scores per thread (about 1024 in all,
//      spread evenly over each thread's entries) gives a value t0 whose share
//      of the samples at or above it is the expected share of sel plus five
//      standard deviations of a binomial count;
//   2. the scores >= t0 ("survivors") are counted per thread (a bitmask) and
//      over the workgroup; when there are at least sel of them (so every
//      score equal to the sel-th largest is one) and no thread holds more than
//      SMAX, each thread keeps its own survivors in registers, still in entry
//      order, so thread order is entry order;
//   3. a value-linear histogram of the survivors between t0 and the max gives
//      the bin of the sel-th largest, whose scores are gathered and ranked
//      (ballots over one wavefront's lanes);
//   4. ordered compaction of the survivors: one workgroup scan of per-thread
//      (greater, equal) counts packed in 16-bit halves.
// A short list for a second, smaller rank (run2) comes from the same
// histogram: the survivors of the bins from that rank's bin upwards,
// compacted in the same scan as the top-sel list (no second ranking).
// Histograms have kFBins bins, few enough that every wavefront scans them on
// its own (no broadcast barrier); cross-lane steps use DPP; passes over all
// scores keep several independent accumulators (one wavefront per SIMD leaves
// no other latency hiding).  When the survivors are too few or too crowded in
// one thread (ties, very small ranges, structured inputs) the radix selection
// on order-preserving keys runs on all scores instead, with the same result:
// the sample only decides how much work the exact steps see.
template <int THREADS, int ITEMS, int SMAX>
struct Filter {
  using Big = Select<THREADS, ITEMS>;
  using Small = Select<THREADS, SMAX>;
  using Mask = typename Big::Mask;
  using SMask = typename Small::Mask;
  static constexpr int kNs = 1024 / THREADS;  // samples per thread
  static_assert(kNs >= 1 && kNs <= 32 && ITEMS % kNs == 0 && ITEMS % 8 == 0, "sampling");
  static_assert(SMAX <= 32, "survivor bitmask");
  static constexpr int kWaves = THREADS / 64;
  static constexpr int kFBins = 256;  // four bins per lane

  struct Shared {
    SelectShared<THREADS> core;          // radix selection state (fallback)
    alignas(16) uint32_t shist[kFBins];  // sample histogram
    alignas(16) uint32_t hist2[kFBins];  // survivor histogram
    alignas(16) float ck[kSmall + 64];   // scores of the threshold bin; 64 lane-private dump slots after them
    uint32_t wsum[kWaves];
    uint32_t wsum2[kWaves];
    float red[2][kWaves];
    uint32_t ncand;
  };

  // Zero what run() expects zeroed; a barrier must follow (block_range has one).
  static __device__ __forceinline__ void zero(Shared& sh) {
    for (int i = threadIdx.x; i < kFBins; i += THREADS) {
      sh.shist[i] = 0;
      sh.hist2[i] = 0;
    }
    if (threadIdx.x == 0) sh.ncand = 0;
  }

  // Min and max of the non-NaN scores of the workgroup (one barrier).
  static __device__ __forceinline__ void block_range(const float (&x)[ITEMS], Shared& sh, float* vmin, float* vmax) {
    const int wave = threadIdx.x >> 6;
    float lo[8], hi[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      lo[a] = x[a];
      hi[a] = x[a];
    }
#pragma unroll
    for (int j = 8; j < ITEMS; ++j) {
      lo[j & 7] = __builtin_fminf(lo[j & 7], x[j]);
      hi[j & 7] = __builtin_fmaxf(hi[j & 7], x[j]);
    }
#pragma unroll
    for (int a = 4; a >= 1; a >>= 1)
#pragma unroll
      for (int b = 0; b < a; ++b) {
        lo[b] = __builtin_fminf(lo[b], lo[b + a]);
        hi[b] = __builtin_fmaxf(hi[b], hi[b + a]);
      }
    const float l = wave_fmin(lo[0]), h = wave_fmax(hi[0]);
    if (lane_id() == 0) {
      sh.red[0][wave] = l;
      sh.red[1][wave] = h;
    }
    __syncthreads();
    float rl = sh.red[0][0], rh = sh.red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      rl = __builtin_fminf(rl, sh.red[0][w]);
      rh = __builtin_fmaxf(rh, sh.red[1][w]);
    }
    *vmin = rl;
    *vmax = rh;
  }

  // Bin (top first) of the r-th largest of a kFBins histogram, found by every
  // wavefront on its own: lane l holds bins 255-4l .. 252-4l.  rank(total)
  // gives r from the histogram total; returns the total, the bin, the count
  // above the bin and the bin's own count (wave-uniform).
  template <typename Rank>
  static __device__ __forceinline__ void hist_find(const uint32_t* h, Rank rank, uint32_t* total, uint32_t* bin,
                                                   uint32_t* above, uint32_t* cnt) {
    const uint32_t lane = lane_id();
    const uint4 x = *reinterpret_cast<const uint4*>(h + kFBins - 4 - 4 * lane);
    const uint32_t c[4] = {x.w, x.z, x.y, x.x};
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(s);
    const uint32_t tot = last_lane(incl);
    const uint32_t r = rank(tot);
    uint32_t excl = incl - s, b = 0, ab = 0, cb = 0;
    bool hit = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!hit && excl < r && excl + c[q] >= r) {
        hit = true;
        b = kFBins - 1 - 4 * lane - q;
        ab = excl;
        cb = c[q];
      }
      excl += c[q];
    }
    const uint64_t bal = __ballot(hit);
    const int src = bal ? __builtin_ctzll(bal) : 0;
    *total = tot;
    *bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), src));
    *above = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ab), src));
    *cnt = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cb), src));
  }

  // The rem-th largest of the n (1 <= rem <= n <= kSmall) scores in ck and
  // how many scores equal to it rank within the first rem, computed by every
  // wavefront.  Up to 64 scores: one per lane, and candidate i is ranked with
  // two ballots (stops at the answer); more: each lane counts over all.
  static __device__ __forceinline__ void rank_small(const float* ck, uint32_t n, uint32_t rem, float* thr,
                                                    uint32_t* take) {
    const uint32_t lane = lane_id();
    if (n <= 64) {
      const float mine = lane < n ? ck[lane] : -__builtin_inff();
      for (uint32_t i = 0; i < n; ++i) {
        const float ci = __uint_as_float(static_cast<uint32_t>(
            __builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(mine)), static_cast<int>(i))));
        const uint32_t gt = static_cast<uint32_t>(__popcll(__ballot(mine > ci)));
        const uint32_t ge = static_cast<uint32_t>(__popcll(__ballot(mine >= ci)));
        if (gt < rem && ge >= rem) {
          *thr = ci;
          *take = rem - gt;
          return;
        }
      }
      *thr = 0.f;  // not reached: some score has rank rem
      *take = 0;
      return;
    }
    constexpr int kQ = kSmall / 64;
    float mk[kQ];
    uint32_t gt[kQ], ge[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      mk[q] = lane + 64 * q < n ? ck[lane + 64 * q] : -__builtin_inff();
      gt[q] = 0;
      ge[q] = 0;
    }
    for (uint32_t i = 0; i < n; ++i) {
      const float e = ck[i];
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        gt[q] += e > mk[q];
        ge[q] += e >= mk[q];
      }
    }
    float tk = 0.f;
    uint32_t tt = 0;
    bool hit = false;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (!hit && lane + 64 * q < n && gt[q] < rem && ge[q] >= rem) {
        hit = true;
        tk = mk[q];
        tt = rem - gt[q];
      }
    const uint64_t bal = __ballot(hit);
    const int src = bal ? __builtin_ctzll(bal) : 0;
    *thr = __uint_as_float(static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(tk)), src)));
    *take = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tt), src));
  }

  // Keeps the sel largest valid scores (1 <= sel <= nvalid = valid scores of
  // the workgroup, vmin / vmax their min and max).  Kept items get slots in
  // entry order: emit(pos, score, entry) on the sampled path, emit_item(j,
  // pos) (item j of this thread) on the radix path.  On the sampled path
  // emit is also called for items that are not kept, with pos == kNoSlot (to
  // be dropped, for instance stored to a dump slot).  src(e) returns the
  // score of entry e.  Ends with a barrier.
  template <typename Src, typename Emit, typename EmitItem>
  static __device__ __forceinline__ void run(const float (&x)[ITEMS], Src src, uint32_t nvalid, uint32_t sel,
                                             float vmin, float vmax, Shared& sh, Emit emit, EmitItem emit_item) {
    float t2;
    uint32_t c2;
    run2(x, src, nvalid, sel, vmin, vmax, sh, emit, emit_item, 0u, [](uint32_t, float, uint32_t) {}, &t2, &c2);
  }

  // run() plus a short list for a second rank sel2 (1 <= sel2 <= sel; 0:
  // none): on the sampled path every survivor in the survivor-histogram bins
  // from the one holding the sel2-th largest score upwards (so at least sel2
  // scores) is emitted again, in entry order, through emit2(pos, score,
  // entry) (also called with pos == kNoSlot for the other survivors); *cnt2 gets their number and *thr2 their smallest score, and since
  // bins are monotone in the score, every valid score >= *thr2 is in the
  // list.  On the radix paths no list is made (*cnt2 = 0xffffffff).  Ends
  // with a barrier.
  template <typename Src, typename Emit, typename EmitItem, typename Emit2>
  static __device__ __forceinline__ void run2(const float (&x)[ITEMS], Src src, uint32_t nvalid, uint32_t sel,
                                              float vmin, float vmax, Shared& sh, Emit emit, EmitItem emit_item,
                                              uint32_t sel2, Emit2 emit2, float* thr2, uint32_t* cnt2) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const uint32_t lane = lane_id();
    const float range = vmax - vmin;
    const float scale = static_cast<float>(kFBins) / range;
    // uniform: every operand is
    bool filt = sel * 4u <= nvalid && vmin < vmax && __builtin_isfinite(vmin) && __builtin_isfinite(vmax) &&
                __builtin_isfinite(range) && __builtin_isfinite(scale);
    float t0 = 0.f;
    if (filt) {
#pragma unroll
      for (int q = 0; q < kNs; ++q) {
        const float v = x[q * (ITEMS / kNs)];
        if (v == v) {
          const int bb = static_cast<int>((v - vmin) * scale);
          atomicAdd(&sh.shist[bb < kFBins - 1 ? bb : kFBins - 1], 1u);
        }
      }
      __syncthreads();
      uint32_t ns, b, ab, cb;
      hist_find(sh.shist, [&](uint32_t tot) {
        const float e = static_cast<float>(sel) * static_cast<float>(tot) / static_cast<float>(nvalid);
        const uint32_t rr = static_cast<uint32_t>(e + 5.f * __builtin_sqrtf(e)) + 4u;
        return rr < tot ? rr : tot;
      }, &ns, &b, &ab, &cb);
      filt = ns >= 64;
      t0 = vmin + static_cast<float>(b) / scale;  // about the lower edge of that bin
    }
    // Survivors: a bitmask per thread (four independent partial masks), the
    // count and an overflow flag (more than SMAX) summed over the workgroup.
    Mask gm = 0;
    if (filt) {
      Mask g4[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) g4[j & 3] |= static_cast<Mask>(x[j] >= t0) << j;
      gm = (g4[0] | g4[1]) | (g4[2] | g4[3]);
    }
    const uint32_t c = Big::popc(gm);
    const uint32_t packed = c | (static_cast<uint32_t>(c > static_cast<uint32_t>(SMAX)) << 20);
    const uint32_t incl = wave_incl_scan(packed);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += sh.wsum[w];
    const uint32_t total = tot & 0xfffffu;
    if (!(filt && total >= sel && (tot >> 20) == 0)) {
      uint32_t keys[ITEMS];
      Mask vm = 0;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        keys[j] = float_key(x[j]);
        vm |= static_cast<Mask>(x[j] == x[j]) << j;
      }
      Big::zero(sh.core);
      __syncthreads();
      uint32_t thr, take, bg = 0, be = 0;
      Big::radix_select(keys, vm, sel, sh.core, &thr, &take);
      Big::compact(keys, vm, thr, take, sh.core, &bg, &be, emit_item);
      *thr2 = 0.f;
      *cnt2 = 0xffffffffu;  // no short list on this path
      return;
    }
    // This thread's survivors, in entry order, into registers (scores read
    // back from LDS: the loads are independent).
    uint32_t ent[SMAX];
    float y[SMAX];
    Mask m = gm;
#pragma unroll
    for (int k = 0; k < SMAX; ++k) {
      const int j = m ? static_cast<int>(Big::ctz(m)) : 0;
      m &= m - 1;
      ent[k] = static_cast<uint32_t>(tid * ITEMS + j);
    }
#pragma unroll
    for (int k = 0; k < SMAX; ++k) {
      const float v = src(ent[k]);
      y[k] = static_cast<uint32_t>(k) < c ? v : __builtin_nanf("");
    }
    const float range2 = vmax - t0;
    const float scale2 = static_cast<float>(kFBins) / range2;
    const bool spread = range2 > 0.f && __builtin_isfinite(range2) && __builtin_isfinite(scale2);  // uniform
    const bool two = sel2 != 0;                                                                   // uniform
    int bn[SMAX];
#pragma unroll
    for (int k = 0; k < SMAX; ++k) bn[k] = -1;
    uint32_t cb2 = 0, ab2 = 0, b2 = 0, b3 = 0;
    if (spread) {
#pragma unroll
      for (int k = 0; k < SMAX; ++k) {
        const int bb = static_cast<int>((y[k] - t0) * scale2);
        bn[k] = static_cast<uint32_t>(k) < c ? (bb < kFBins - 1 ? bb : kFBins - 1) : -1;
        if (bn[k] >= 0) atomicAdd(&sh.hist2[bn[k]], 1u);
      }
      __syncthreads();
      uint32_t n2, ab3, cb3;
      hist_find(sh.hist2, [&](uint32_t) { return sel; }, &n2, &b2, &ab2, &cb2);
      if (two) hist_find(sh.hist2, [&](uint32_t) { return sel2; }, &n2, &b3, &ab3, &cb3);
    }
    float thr;
    uint32_t take;
    const bool crowded = !spread || cb2 > static_cast<uint32_t>(kSmall);  // uniform
    if (crowded) {
      // One value or a crowded bin: radix passes over the survivors' keys.
      uint32_t k2[SMAX];
      SMask v2 = 0;
#pragma unroll
      for (int k = 0; k < SMAX; ++k) {
        k2[k] = float_key(y[k]);
        v2 |= static_cast<SMask>(static_cast<uint32_t>(k) < c) << k;
      }
      Big::zero(sh.core);
      __syncthreads();
      uint32_t tk;
      Small::radix_select(k2, v2, sel, sh.core, &tk, &take);
      thr = key_float(tk);
    } else {
      // Gather the threshold bin's scores (one LDS atomic per wavefront
      // reserves the space); every wavefront then ranks them.
      SMask m2 = 0;
#pragma unroll
      for (int k = 0; k < SMAX; ++k) m2 |= static_cast<SMask>(bn[k] == static_cast<int>(b2)) << k;
      const uint32_t c2 = Small::popc(m2);
      const uint32_t in2 = wave_incl_scan(c2);
      uint32_t base = 0;
      if (lane == 63 && in2 != 0) base = atomicAdd(&sh.ncand, in2);
      base = last_lane(base);
      if (last_lane(in2) != 0)
        scatter_flagged<SMAX>(m2, base + in2 - c2, kSmall, kSmall + lane, sh.ck, [&](int k) { return y[k]; });
      __syncthreads();
      rank_small(sh.ck, cb2, sel - ab2, &thr, &take);
    }
    // Ordered compaction of the survivors for both lists with one barrier:
    // (greater, equal) counts packed in 16-bit halves for the top-sel list,
    // the count in bins >= b3 for the short one (with their smallest score),
    // two wavefront scans.
    const bool list2 = two && !crowded;  // uniform
    SMask gtm = 0, eqm = 0, gm2 = 0;
    float lo2 = __builtin_inff();
#pragma unroll
    for (int k = 0; k < SMAX; ++k) {
      gtm |= static_cast<SMask>(y[k] > thr) << k;
      eqm |= static_cast<SMask>(y[k] == thr) << k;
      const bool in2 = list2 && bn[k] >= static_cast<int>(b3);
      gm2 |= static_cast<SMask>(in2) << k;
      lo2 = in2 ? __builtin_fminf(lo2, y[k]) : lo2;
    }
    const uint32_t packed1 = (Small::popc(eqm) << 16) | Small::popc(gtm);
    const uint32_t q2 = Small::popc(gm2);
    const uint32_t pin = wave_incl_scan(packed1);
    const uint32_t qin = wave_incl_scan(q2);
    const float lo2w = wave_fmin(lo2);
    if (lane == 63) {
      sh.core.wsum[wave] = pin;
      sh.wsum2[wave] = qin;
      sh.red[0][wave] = lo2w;
    }
    __syncthreads();
    uint32_t excl = pin - packed1, qpos = qin - q2, qtot = 0;
    float tv2 = __builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      excl += w < wave ? sh.core.wsum[w] : 0u;
      qpos += w < wave ? sh.wsum2[w] : 0u;
      qtot += sh.wsum2[w];
      tv2 = __builtin_fminf(tv2, sh.red[0][w]);
    }
    const uint32_t gt0 = excl & 0xffffu, eq0 = excl >> 16;
    uint32_t keq = take > eq0 ? take - eq0 : 0u;
    SMask km = gtm, em = eqm;
    while (keq > 0 && em) {
      const SMask lb = em & (0 - em);
      km |= lb;
      em ^= lb;
      --keq;
    }
    uint32_t slot = gt0 + (eq0 < take ? eq0 : take);
    // Every survivor slot calls the emitters, branch-free: a slot that is
    // not kept gets kNoSlot (per-item exec-mask branches cost more than the
    // stores they skip).
#pragma unroll
    for (int k = 0; k < SMAX; ++k) {
      const bool kp = Small::bit(km, k);
      emit(kp ? slot : kNoSlot, y[k], ent[k]);
      slot += kp;
    }
    if (two) {
#pragma unroll
      for (int k = 0; k < SMAX; ++k) {
        const bool kp = Small::bit(gm2, k);
        emit2(kp ? qpos : kNoSlot, y[k], ent[k]);
        qpos += kp;
      }
    }
    __syncthreads();
    *thr2 = tv2;
    *cnt2 = list2 ? qtot : 0xffffffffu;
  }

};

}  // namespace sel
}  // namespace csa
