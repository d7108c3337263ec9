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
constexpr int kMaxMergeParts = 256;  // part counts cached in LDS by the merge
constexpr int kStage = 2048;         // outputs up to this size are staged in LDS, then stored coalesced
using Sel = sel::Select<kThreads, kItems>;
using Filt = sel::Filter<kThreads, kItems, 8>;
using sel::lane_id;
using sel::wave_incl_scan;

struct Shared {
  Filt::Shared fs;
  int32_t pcnt[kMaxMergeParts];
  int32_t si[kStage];  // staged output: payload (entry or index) and score
  float sv[kStage];
};

__device__ __forceinline__ int64_t row_visible(const TopkArgs& a, int64_t row) {
  const int64_t tpos = a.n_ctx - a.T + row % a.T;
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
  if (cnt <= 0) {
    if (threadIdx.x == 0) *cc = 0;
    return;
  }
  Filt::zero(sh.fs);
  const float* s = a.score + lrow * a.ld + base;
  float* ov = cval + (lrow * nparts + part) * cap;
  int32_t* oi = cidx + (lrow * nparts + part) * cap;
  const int tid = threadIdx.x;
  const int i0 = tid * kItems;  // this thread's entries i0 .. i0+31 of the part
  float v[kItems];
  const int nvalid = cnt - i0 <= 0 ? 0 : (cnt - i0 >= kItems ? kItems : static_cast<int>(cnt - i0));
  if (nvalid == kItems && (reinterpret_cast<uintptr_t>(s) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(s + i0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const float t = s[j < nvalid ? i0 + j : 0];  // in range: the part has at least one entry
      v[j] = j < nvalid ? t : __builtin_nanf("");
    }
  }
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
  float vmin, vmax;
  Filt::block_range(v, sh.fs, &vmin, &vmax);
  const uint32_t ncnt = static_cast<uint32_t>(cnt), ucap = static_cast<uint32_t>(cap);
  auto pay = [&](int j) { return static_cast<uint32_t>(i0 + j); };
  if (cap <= kStage) {  // stage the kept entries in LDS, then store them coalesced
    Filt::run(
        v, pay, ncnt, ucap, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t e) {
          sh.si[pos] = static_cast<int>(e);
          sh.sv[pos] = val;
        },
        [&](int j, uint32_t pos) {
          sh.si[pos] = i0 + j;
          sh.sv[pos] = s[i0 + j];
        });
    for (int i = tid; i < cap; i += kThreads) {
      ov[i] = sh.sv[i];
      oi[i] = static_cast<int32_t>(base + sh.si[i]);
    }
  } else {
    Filt::run(
        v, pay, ncnt, ucap, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t e) {
          ov[pos] = val;
          oi[pos] = static_cast<int32_t>(base + e);
        },
        [&](int j, uint32_t pos) {
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
                                                              const int32_t* cidx, const int32_t* ccnt, bool fused) {
  __shared__ Shared sh;
  __shared__ int wtot[kThreads / 64];
  const int64_t lrow = blockIdx.x;
  if (!fused && merge_trivial(a, lrow)) return;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;
  const int ns = nparts * cap;
  const float* rv = cval + lrow * ns;
  const int32_t* ri = cidx + lrow * ns;
  const int32_t* rc = ccnt + lrow * nparts;
  Filt::zero(sh.fs);
  static_assert(kMaxMergeParts <= kThreads, "one part count per thread");
  int pc = 0;
  if (tid < nparts) {
    pc = rc[tid];
    sh.pcnt[tid] = pc;
  }
  pc = static_cast<int>(sel::wave_sum(static_cast<uint32_t>(pc)));
  if (lane_id() == 0) wtot[tid >> 6] = pc;
  __syncthreads();
  int total = 0;  // valid candidates of the row
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) total += wtot[w];
  const uint32_t ucap = static_cast<uint32_t>(cap);
  const uint32_t magic = static_cast<uint32_t>((0x100000000ull + ucap - 1) / ucap);
  float v[kItems];
  uint32_t ix[kItems];
  const int s0 = tid * kItems;
  if (s0 + kItems <= ns && ((reinterpret_cast<uintptr_t>(rv + s0) | reinterpret_cast<uintptr_t>(ri + s0)) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(rv + s0 + 4 * q);
      const u32x4 y = *reinterpret_cast<const u32x4*>(ri + s0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[4 * q + e] = x[e];
        ix[4 * q + e] = y[e];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int sc = s0 + j < ns ? s0 + j : ns - 1;
      v[j] = rv[sc];
      ix[j] = static_cast<uint32_t>(ri[sc]);
    }
  }
  // Slots past their part's count hold no candidate: NaN (never selected).
  // Branch-free on purpose (the part count is read for every slot, clamped
  // in range): a conditional store into the register array here has been
  // compiled into code that loses the store for the first item.
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int sl = s0 + j;
    const int sc = sl < ns ? sl : ns - 1;
    const uint32_t pp = __umulhi(static_cast<uint32_t>(sc), magic);
    const int pcount = sh.pcnt[pp];
    const bool ok = (sl < ns) & (static_cast<int>(static_cast<uint32_t>(sc) - pp * ucap) < pcount);
    v[j] = ok ? v[j] : __builtin_nanf("");
  }
  if (total <= a.k) {  // every valid candidate is kept, in slot order; -1 padding after them
    for (int64_t i = total + tid; i < a.k; i += kThreads) {
      o[i] = -1;
      if (os) os[i] = -INFINITY;
    }
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) c += v[j] == v[j];
    const uint32_t incl = wave_incl_scan(c);
    if (lane_id() == 63) sh.fs.core.wsum[tid >> 6] = incl;  // wtot may still be read
    __syncthreads();
    uint32_t pos = incl - c;
    for (int w = 0; w < (tid >> 6); ++w) pos += sh.fs.core.wsum[w];
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (v[j] == v[j]) {
        o[pos] = static_cast<int32_t>(ix[j]);
        if (os) os[pos] = v[j];
        ++pos;
      }
    return;
  }
  const uint32_t uk = static_cast<uint32_t>(a.k);
  float vmin, vmax;
  Filt::block_range(v, sh.fs, &vmin, &vmax);
  auto pay = [&](int j) { return ix[j]; };
  if (a.k <= kStage) {  // stage the kept candidates in LDS, then store coalesced
    Filt::run(
        v, pay, static_cast<uint32_t>(total), uk, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t idx) {
          sh.si[pos] = static_cast<int32_t>(idx);
          sh.sv[pos] = val;
        },
        [&](int j, uint32_t pos) {
          sh.si[pos] = ri[s0 + j];
          sh.sv[pos] = rv[s0 + j];
        });
    for (int i = tid; i < a.k; i += kThreads) {
      o[i] = sh.si[i];
      if (os) os[i] = sh.sv[i];
    }
  } else {
    Filt::run(
        v, pay, static_cast<uint32_t>(total), uk, vmin, vmax, sh.fs,
        [&](uint32_t pos, float val, uint32_t idx) {
          o[pos] = static_cast<int32_t>(idx);
          if (os) os[pos] = val;
        },
        [&](int j, uint32_t pos) {
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
  return launch_topk_merge(a, np, cap, cval, cidx, ccnt, false, s);
}

hipError_t launch_topk_merge(const TopkArgs& a, int64_t np, int64_t cap, const float* cval, const int32_t* cidx,
                             const int32_t* ccnt, bool fused, hipStream_t s) {
  if (a.nrows == 0 || a.k == 0) return hipSuccess;
  if (np * cap <= kPart && np <= kMaxMergeParts) {
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a,
                       static_cast<int>(np), static_cast<int>(cap), cval, cidx, ccnt, fused);
  } else {
    if (fused) return hipErrorInvalidValue;  // the fused path only takes the fast merge
    hipLaunchKernelGGL(topk_merge_general, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a, np, cap,
                       cval, cidx, ccnt);
  }
  return hipGetLastError();
}

}  // namespace csa
