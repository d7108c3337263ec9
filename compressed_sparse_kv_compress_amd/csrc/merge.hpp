// Per-row merge stages of the exact top-k, written for any workgroup size
// (the stand-alone merge kernel runs them with 512 threads).
//
// Method: shareware.cn Hybrid Attention article, section 六 (score, then keep
// the top-k entries); aimodeling.com news item, CSA paragraph (1024 per
// query).  Equal scores (-0 == +0) go to the lower entry index; the kept
// indices are written in ascending order, -1 padded.
#pragma once
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace csa {
namespace mrg {

constexpr int kStage = 2048;  // outputs up to this size are staged in LDS, then stored coalesced
constexpr int32_t kWholePart = -2;  // list count of a part kept whole: its list is its candidate set
constexpr int kSlots = 16384;  // candidate slots one merge holds

// A tile of up to THREADS * ITEMS scores staged in LDS: thread t owns entries
// t*ITEMS .. t*ITEMS+ITEMS-1, stored with 4 pad words after every ITEMS
// entries so that the owners' 16-byte reads of their own entries hit distinct
// bank groups.
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

// Visible entries of launch row `row` (positions from the end of its sequence).
__device__ __forceinline__ int64_t row_visible(const TopkArgs& a, int64_t row) {
  SeqLayout l;
  l.lens = a.lens;
  const int64_t tpos = seq_len(l, a.n_ctx, a.T, row / a.T) - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  return nv < 0 ? 0 : nv;
}

// Merge of one row's candidates by a THREADS-thread workgroup.
template <int THREADS>
struct Merge {
  static constexpr int ITEMS = kSlots / THREADS;
  static constexpr int SMAX = ITEMS <= 32 ? 16 : 24;  // survivors a thread keeps in registers
  static constexpr int kWaves = THREADS / 64;
  using T = Tile<THREADS, ITEMS>;
  using F = sel::Filter<THREADS, ITEMS, SMAX>;
  struct Shared {
    typename F::Shared fs;
    int32_t si[kStage + 64];  // 64 lane-private dump slots at the end
    float sv[kStage + 64];
    alignas(16) float stage[T::kFloats];
    int wtot[kWaves];
  };

  // Merge from per-part short lists.  Part p's list holds, in index order,
  // every entry of the part with a score >= lthr[p] (at least the part's
  // lrank largest); lcnt[p] = -1 means no list.  U, the union of the lists in
  // part (= index) order, has at most THREADS * UITEMS entries.  With theta_U
  // the k-th largest of U (a subset of the row, so theta_U <= the row's k-th
  // largest theta), an entry of the row's top-k has a score >= theta >=
  // theta_U; when every lthr[p] <= theta_U that score is >= its part's
  // threshold, so the entry is in U and the top-k of U is the row's.  Returns
  // false (nothing written) when a list is missing, U holds fewer than k or
  // more than THREADS * UITEMS entries, or some lthr[p] > theta_U.  nparts <=
  // THREADS.  lthr == nullptr: every list is its part's whole candidate set
  // (nothing to test).  lcnt[p] == kWholePart: part p was kept whole (at most
  // k entries, no list); its list is its candidate set, the ccnt[p] entries
  // at cval / cidx + p * ccap, all of them (threshold -inf).
  //
  // U is read in one of two ways.  Usually every list holds at most
  // S = THREADS * UITEMS / nparts entries: then U stays a padded grid, entry
  // e = p * S + j being slot j of part p's list (valid for j < lcnt[p]),
  // requested together with the counts, so one memory round trip brings it
  // in; grid order is still index order.  Otherwise U is packed into LDS by
  // a binary search of each entry's part over the list offsets (a second
  // round trip, any list lengths).
  template <int UITEMS>
  static __device__ __forceinline__ bool lists(int k, int nparts, const float* lval, const int32_t* lidx, const int32_t* lcnt,
                               const float* lthr, int64_t lcap, Shared& sh, int32_t* o, float* os,
                               const float* cval = nullptr, const int32_t* cidx = nullptr,
                               const int32_t* ccnt = nullptr, int64_t ccap = 0) {
    static_assert(2 * THREADS * UITEMS <= T::kFloats, "the union fits the stage");
    using USel = sel::Select<THREADS, UITEMS>;
    constexpr int kU = THREADS * UITEMS;
    if (k > kStage / 2) return false;  // the output is staged in half of si (past the list offsets)
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    // counts, thresholds and candidate counts are all requested at once
    int lc = tid < nparts ? lcnt[tid] : 0;
    const float lt0 = tid < nparts && lthr ? lthr[tid] : -INFINITY;
    const int cc = tid < nparts && ccnt ? ccnt[tid] : 0;
    // the padded grid's loads go out with the counts (slots past a list's
    // count are read but never used; every address stays in part p's lcap slots)
    const int S = kU / (nparts > 0 ? nparts : 1);
    float tv[UITEMS];
    int32_t tx[UITEMS];
    // 16-byte loads when a thread's slots are whole aligned vectors of one
    // part's list (S a multiple of UITEMS, lists 16-byte aligned)
    const bool vec = S % UITEMS == 0 && lcap % 4 == 0 && S <= lcap &&
                     ((reinterpret_cast<uintptr_t>(lval) | reinterpret_cast<uintptr_t>(lidx)) & 15) == 0;  // uniform
    if (vec) {
      static_assert(UITEMS % 4 == 0, "whole vectors");
      const int e0 = tid * UITEMS;
      const int p = e0 / S;
      const int64_t at = static_cast<int64_t>(p < nparts ? p : 0) * lcap + (e0 - p * S);
#pragma unroll
      for (int q = 0; q < UITEMS / 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(lval + at + 4 * q);
        const u32x4 x = *reinterpret_cast<const u32x4*>(lidx + at + 4 * q);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          tv[4 * q + u] = v[u];
          tx[4 * q + u] = static_cast<int32_t>(x[u]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < UITEMS; ++j) {
        const int e = tid * UITEMS + j;
        const int p = e / S;
        const int jj = e - p * S;
        const int64_t at = static_cast<int64_t>(p < nparts ? p : 0) * lcap + (jj < lcap ? jj : 0);
        tv[j] = lval[at];
        tx[j] = lidx[at];
      }
    }
    const bool whole = lc == kWholePart && ccnt != nullptr;
    if (whole) lc = cc;
    const float lt = whole ? -INFINITY : lt0;
    // per wave: any missing list, the lists' total, the largest threshold,
    // the longest list (a whole part counts as too long for the grid)
    const uint32_t neg = static_cast<uint32_t>(__popcll(__ballot(lc < 0)));
    const uint32_t cnt = static_cast<uint32_t>(lc > 0 ? lc : 0);
    const uint32_t incl = sel::wave_incl_scan(cnt);
    const float vmax_w = wave_max(lt);
    const uint32_t cmax_w = sel::wave_max(whole ? 0xffffffffu : cnt);
    uint32_t* uoff = reinterpret_cast<uint32_t*>(sh.si);  // list offsets in U (<= THREADS parts)
    int32_t* ucnt = sh.si + THREADS;                        // list lengths
    if (sel::lane_id() == 63) {
      sh.fs.wsum[wave] = incl;
      sh.fs.red[0][wave] = vmax_w;
      sh.fs.core.red[0][wave] = neg;
      sh.fs.core.red[1][wave] = cmax_w;
    }
    __syncthreads();
    uint32_t before = 0, total = 0, nneg = 0, cmax = 0;
    float vmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      before += w < wave ? sh.fs.wsum[w] : 0u;
      total += sh.fs.wsum[w];
      nneg += sh.fs.core.red[0][w];
      vmax = fmaxf(vmax, sh.fs.red[0][w]);
      cmax = cmax > sh.fs.core.red[1][w] ? cmax : sh.fs.core.red[1][w];
    }
    if (nneg != 0 || total < static_cast<uint32_t>(k) || total > static_cast<uint32_t>(kU)) {
      __syncthreads();  // the LDS reads above are done before the caller reuses it
      return false;
    }
    if (tid < nparts) {
      uoff[tid] = before + incl - cnt;
      ucnt[tid] = whole ? -static_cast<int32_t>(cnt) : static_cast<int32_t>(cnt);  // negative: a whole part
    }
    __syncthreads();
    const bool grid = cmax <= static_cast<uint32_t>(S) && static_cast<int64_t>(S) <= lcap;  // uniform
    uint32_t keys[UITEMS];
    typename USel::Mask vm = 0;
    if (grid) {
#pragma unroll
      for (int j = 0; j < UITEMS; ++j) {
        const int e = tid * UITEMS + j;
        const int p = e / S;
        const int jj = e - p * S;
        const bool ok = p < nparts && jj < ucnt[p < nparts ? p : 0];
        keys[j] = float_key(tv[j]);
        vm |= static_cast<typename USel::Mask>(ok) << j;
      }
    } else {
      // U packed into LDS (values, then indices).  Entry e of U is entry
      // e - uoff[p] of part p's list (of its candidate set for a whole part),
      // p the last part with uoff[p] <= e (empty parts share their
      // successor's offset, so p is the part that holds e); each thread
      // issues all its loads before its stores.  U holds at most kU entries
      // (checked above), so the arithmetic fits 32 bits.
      float* uval = sh.stage;
      int32_t* uidx = reinterpret_cast<int32_t*>(sh.stage + kU);
#pragma unroll
      for (int r = 0; r < UITEMS; ++r) {
        const uint32_t e = static_cast<uint32_t>(r * THREADS + tid);
        const uint32_t ec = e < total ? e : 0u;
        int lo = 0, hi = nparts - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (uoff[mid] <= ec) lo = mid;
          else hi = mid - 1;
        }
        const int64_t jj = static_cast<int64_t>(ec - uoff[lo]);
        const bool wp = ucnt[lo] < 0;  // a whole part (only when ccnt was given)
        const float* vb = wp ? cval : lval;
        const int32_t* ib = wp ? cidx : lidx;
        const int64_t at = static_cast<int64_t>(lo) * (wp ? ccap : lcap) + jj;
        tv[r] = vb[at];
        tx[r] = ib[at];
      }
#pragma unroll
      for (int r = 0; r < UITEMS; ++r) {
        const uint32_t e = static_cast<uint32_t>(r * THREADS + tid);
        if (e < total) {
          uval[e] = tv[r];
          uidx[e] = tx[r];
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < UITEMS; ++j) {
        const uint32_t u = static_cast<uint32_t>(tid * UITEMS + j);
        tv[j] = uval[u < total ? u : 0];
        tx[j] = uidx[u < total ? u : 0];
        keys[j] = float_key(tv[j]);
        vm |= static_cast<typename USel::Mask>(u < total) << j;
      }
    }
    USel::zero(sh.fs.core);
    __syncthreads();
    uint32_t thr, take;
    USel::radix_select(keys, vm, static_cast<uint32_t>(k), sh.fs.core, &thr, &take);
    if (vmax > key_float(thr)) {  // uniform: some part's list may miss row top-k entries
      __syncthreads();
      return false;
    }
    uint32_t bg = 0, be = 0;
    // outputs staged in sh.sv / sh.si past the list offsets (k <= kStage / 2 here)
    USel::compact(keys, vm, thr, take, sh.fs.core, &bg, &be, [&](int j, uint32_t pos) {
      sh.sv[pos] = tv[j];
      sh.si[pos + kStage / 2] = tx[j];
    });
    for (int i = tid; i < k; i += THREADS) {
      o[i] = sh.si[i + kStage / 2];
      if (os) os[i] = sh.sv[i];
    }
    return true;
  }

  // Merge over nparts * cap <= kSlots candidate slots (part order = index
  // order; slots past a part's count hold NaN).  Every valid candidate is
  // kept when there are at most k of them.
  static __device__ __forceinline__ void full(int k, int nparts, int cap, const float* rv, const int32_t* ri, const int32_t* rc,
                              Shared& sh, int32_t* o, float* os) {
    const int tid = threadIdx.x;
    const int ns = nparts * cap;
    // The candidate loads go out first; the part counts are summed meanwhile.
    const typename T::Loads ld = T::load(rv, ns);
    F::zero(sh.fs);
    const int pc = static_cast<int>(sel::wave_sum(static_cast<uint32_t>(tid < nparts ? rc[tid] : 0)));
    if (sel::lane_id() == 0) sh.wtot[tid >> 6] = pc;
    float v[ITEMS];
    T::store(ld, sh.stage, v);  // its barrier also publishes wtot
    int total = 0;  // valid candidates of the row
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += sh.wtot[w];
    const int s0 = tid * ITEMS;
    if (total <= k) {  // every valid candidate is kept, in slot order; -1 padding after them
      for (int i = total + tid; i < k; i += THREADS) {
        o[i] = -1;
        if (os) os[i] = -INFINITY;
      }
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) c += v[j] == v[j];
      const uint32_t incl = sel::wave_incl_scan(c);
      if (sel::lane_id() == 63) sh.fs.core.wsum[tid >> 6] = incl;
      __syncthreads();
      uint32_t pos = incl - c;
      for (int w = 0; w < (tid >> 6); ++w) pos += sh.fs.core.wsum[w];
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if (v[j] == v[j]) {
          o[pos] = ri[s0 + j];
          if (os) os[pos] = v[j];
          ++pos;
        }
      return;
    }
    const uint32_t uk = static_cast<uint32_t>(k);
    float vmin, vmax;
    F::block_range(v, sh.fs, &vmin, &vmax);
    auto src = [&](uint32_t e) { return sh.stage[T::pos(static_cast<int>(e))]; };
    if (k <= kStage) {  // stage the kept candidates in LDS, then store coalesced
      F::run(
          v, src, static_cast<uint32_t>(total), uk, vmin, vmax, sh.fs,
          [&](uint32_t pos, float val, uint32_t e) {
            const uint32_t p = pos != sel::kNoSlot ? pos : kStage + sel::lane_id();
            sh.si[p] = static_cast<int32_t>(e);
            sh.sv[p] = val;
          },
          [&](int j, uint32_t pos) {
            sh.si[pos] = s0 + j;
            sh.sv[pos] = sh.stage[T::pos(s0 + j)];
          });
      for (int i = tid; i < k; i += THREADS) {
        o[i] = ri[sh.si[i]];
        if (os) os[i] = sh.sv[i];
      }
    } else {
      F::run(
          v, src, static_cast<uint32_t>(total), uk, vmin, vmax, sh.fs,
          [&](uint32_t pos, float val, uint32_t e) {
            if (pos == sel::kNoSlot) return;
            o[pos] = ri[e];
            if (os) os[pos] = val;
          },
          [&](int j, uint32_t pos) {
            o[pos] = ri[s0 + j];
            if (os) os[pos] = sh.stage[T::pos(s0 + j)];
          });
    }
  }
};

}  // namespace mrg
}  // namespace csa
