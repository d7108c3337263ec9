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
//   1. part kernel: the row is cut into parts of 16384 scores; one 1024-thread
//      workgroup holds a part in registers (16 consecutive scores per thread),
//      selects the part's own top-min(k, part) with LDS histogram passes of up
//      to 11 bits that start below the common bit prefix of the part's keys,
//      and writes the kept (score, index) pairs in index order.  Any entry of the row's top-k is in its part's top-k, ties
//      included, because fewer entries beat it inside the part than in the
//      whole row.
//   2. merge kernel: one workgroup per row runs the same selection over the
//      concatenated part candidates (part order = index order) and compacts
//      the winners in order.
// Ordered compaction uses one 64-bit workgroup scan per tile (strictly
// greater count in the low word, threshold-equal count in the high word), so
// the lower-index tie rule is exact and the output is sorted without a sort.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 16;
constexpr int64_t kPart = static_cast<int64_t>(kThreads) * kItems;  // 16384

struct Shared {
  uint32_t hist[2048];
  uint64_t scan[2 * kWaves];
  uint32_t red[kWaves];
  uint32_t sel_bin, sel_above;
};

// Inclusive scan of one 64-bit value per thread across the workgroup.
__device__ __forceinline__ uint64_t block_scan_incl(uint64_t v, Shared& sh, uint64_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh.scan[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint64_t w = lane < kWaves ? sh.scan[lane] : 0;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const uint64_t y = __shfl_up(w, o, 64);
      if (lane >= o) w += y;
    }
    if (lane < kWaves) sh.scan[kWaves + lane] = w;
  }
  __syncthreads();
  const uint64_t before = wave ? sh.scan[kWaves + wave - 1] : 0;
  *total = sh.scan[2 * kWaves - 1];
  __syncthreads();
  return v + before;
}

__device__ __forceinline__ uint32_t block_min(uint32_t v, Shared& sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t y = __shfl_xor(v, o, 64);
    v = y < v ? y : v;
  }
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = sh.red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = sh.red[w] < r ? sh.red[w] : r;
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, Shared& sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t y = __shfl_xor(v, o, 64);
    v = y > v ? y : v;
  }
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = sh.red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = sh.red[w] > r ? sh.red[w] : r;
  __syncthreads();
  return r;
}

// Radix select over the valid keys held in registers by the workgroup
// (keys[j] valid iff bit j of vmask is set).  Finds the key of the sel-th
// largest (1-based) and how many keys equal to it are kept (the
// lowest-indexed ones).
__device__ __forceinline__ void radix_select(const uint32_t* keys, uint32_t vmask, uint32_t sel, Shared& sh,
                                             uint32_t* thr_out, uint32_t* take_eq_out) {
  const int tid = threadIdx.x;
  // The valid keys share every bit above the highest bit where their min and
  // max differ; histogramming starts just below that common prefix, so the
  // first pass spreads concentrated scores over all bins instead of piling
  // them onto a few (LDS atomics to one bin serialise).
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kItems; ++j)
    if ((vmask >> j) & 1u) {
      kmin = keys[j] < kmin ? keys[j] : kmin;
      kmax = keys[j] > kmax ? keys[j] : kmax;
    }
  kmin = block_min(kmin, sh);
  kmax = block_max(kmax, sh);
  const uint32_t diff = kmin ^ kmax;
  uint32_t prefix = diff ? (kmax & ~((2u << (31 - __clz(diff))) - 1u)) : kmax;
  uint32_t mask = diff ? ~((2u << (31 - __clz(diff))) - 1u) : 0xffffffffu;
  uint32_t remaining = sel;
  int top = diff ? 31 - __clz(diff) : -1;  // highest undecided bit
  while (top >= 0) {
    const int width = top + 1 < 11 ? top + 1 : 11;
    const int shift = top + 1 - width;
    const int nb = 1 << width;
    for (int i = tid; i < 2048; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (((vmask >> j) & 1u) && (keys[j] & mask) == prefix) atomicAdd(&sh.hist[(keys[j] >> shift) & (nb - 1)], 1u);
    __syncthreads();
    // Scan bins from the top: thread i owns bins nb-1-2i and nb-2-2i.
    const int b0 = nb - 1 - 2 * tid, b1 = nb - 2 - 2 * tid;
    const uint32_t c0 = b0 >= 0 ? sh.hist[b0] : 0, c1 = b1 >= 0 ? sh.hist[b1] : 0;
    uint64_t tot;
    const uint64_t incl = block_scan_incl(static_cast<uint64_t>(c0) + c1, sh, &tot);
    const uint64_t excl = incl - c0 - c1;
    if (b0 >= 0 && excl < remaining && excl + c0 >= remaining) {
      sh.sel_bin = static_cast<uint32_t>(b0);
      sh.sel_above = static_cast<uint32_t>(excl);
    }
    if (b1 >= 0 && excl + c0 < remaining && excl + c0 + c1 >= remaining) {
      sh.sel_bin = static_cast<uint32_t>(b1);
      sh.sel_above = static_cast<uint32_t>(excl + c0);
    }
    __syncthreads();
    prefix |= sh.sel_bin << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    remaining -= sh.sel_above;
    __syncthreads();
    top = shift - 1;
  }
  *thr_out = prefix;
  *take_eq_out = remaining;
}

// Ordered compaction of one tile: thread t holds items t*kItems .. +kItems-1
// of the tile (valid iff bit j of vmask is set).  Kept items get consecutive
// output slots in item order, after *base_gt / *base_eq earlier kept items.
template <typename Emit>
__device__ __forceinline__ void compact_tile(const uint32_t* keys, uint32_t vmask, uint32_t thr, uint64_t take_eq,
                                             Shared& sh, uint64_t* base_gt, uint64_t* base_eq, Emit emit) {
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const bool ok = (vmask >> j) & 1u;
    ngt += ok && keys[j] > thr;
    neq += ok && keys[j] == thr;
  }
  uint64_t tot;
  const uint64_t packed = (static_cast<uint64_t>(neq) << 32) | ngt;
  const uint64_t excl = block_scan_incl(packed, sh, &tot) - packed;
  uint64_t gt_before = *base_gt + (excl & 0xffffffffu);
  uint64_t eq_before = *base_eq + (excl >> 32);
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    if ((vmask >> j) & 1u) {
      const bool gt = keys[j] > thr;
      const bool eq = keys[j] == thr;
      if (gt || (eq && eq_before < take_eq)) emit(j, gt_before + (eq_before < take_eq ? eq_before : take_eq));
      gt_before += gt;
      eq_before += eq;
    }
  }
  *base_gt += tot & 0xffffffffu;
  *base_eq += tot >> 32;
}

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
  const float* s = a.score + lrow * a.ld + base;
  float* ov = cval + (lrow * nparts + part) * cap;
  int32_t* oi = cidx + (lrow * nparts + part) * cap;
  const int64_t i0 = static_cast<int64_t>(threadIdx.x) * kItems;
  const int nvalid = static_cast<int>(cnt - i0 < 0 ? 0 : (cnt - i0 > kItems ? kItems : cnt - i0));
  float v[kItems];
  uint32_t keys[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    v[j] = j < nvalid ? s[i0 + j] : 0.f;
    keys[j] = float_key(v[j]);
  }
  if (cnt <= cap) {  // the whole part is kept
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (j < nvalid) {
        ov[i0 + j] = v[j];
        oi[i0 + j] = static_cast<int32_t>(base + i0 + j);
      }
    if (threadIdx.x == 0) *cc = static_cast<int32_t>(cnt);
    return;
  }
  uint32_t thr, take_eq;
  const uint32_t vmask = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
  radix_select(keys, vmask, static_cast<uint32_t>(cap), sh, &thr, &take_eq);
  uint64_t bg = 0, be = 0;
  compact_tile(keys, vmask, thr, take_eq, sh, &bg, &be, [&](int j, uint64_t pos) {
    ov[pos] = v[j];
    oi[pos] = static_cast<int32_t>(base + i0 + j);
  });
  if (threadIdx.x == 0) *cc = static_cast<int32_t>(cap);
}

// Stage 2: per-row merge of the part candidates.
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(TopkArgs a, int64_t nparts, int64_t cap,
                                                              const float* cval, const int32_t* cidx,
                                                              const int32_t* ccnt) {
  __shared__ Shared sh;
  const int64_t lrow = blockIdx.x;
  const int64_t nv = row_visible(a, a.row0 + lrow);
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;
  if (nv <= a.k) {
    const float* s = a.score + lrow * a.ld;
    for (int64_t i = tid; i < a.k; i += kThreads) {
      o[i] = i < nv ? static_cast<int32_t>(i) : -1;
      if (os) os[i] = i < nv ? s[i] : -INFINITY;
    }
    return;
  }
  // Slots: part p, entry j < ccnt[p]; slot order is index order.
  const int64_t nslots = nparts * cap;
  const float* rv = cval + lrow * nparts * cap;
  const int32_t* ri = cidx + lrow * nparts * cap;
  const int32_t* rc = ccnt + lrow * nparts;
  auto slot_valid = [&](int64_t sl) { return sl < nslots && (sl % cap) < rc[sl / cap]; };

  if (nslots <= kPart) {
    // Fast path: every candidate slot fits one register tile.
    const int64_t i0 = static_cast<int64_t>(tid) * kItems;
    uint32_t keys[kItems];
    float v[kItems];
    int32_t ix[kItems];
    uint32_t vmask = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int64_t sl = i0 + j;
      const bool ok = slot_valid(sl);
      vmask |= static_cast<uint32_t>(ok) << j;
      v[j] = ok ? rv[sl] : 0.f;
      ix[j] = ok ? ri[sl] : 0;
      keys[j] = float_key(v[j]);
    }
    uint32_t thr, take_eq;
    radix_select(keys, vmask, static_cast<uint32_t>(a.k), sh, &thr, &take_eq);
    uint64_t bg = 0, be = 0;
    compact_tile(keys, vmask, thr, take_eq, sh, &bg, &be, [&](int j, uint64_t pos) {
      o[pos] = ix[j];
      if (os) os[pos] = v[j];
    });
    return;
  }

  // General path (many candidates): histogram passes over the slots in L2.
  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(a.k);
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    for (int i = tid; i < 2048; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int64_t sl = tid; sl < nslots; sl += kThreads) {
      if (!slot_valid(sl)) continue;
      const uint32_t key = float_key(rv[sl]);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    const int b0 = nb - 1 - 2 * tid, b1 = nb - 2 - 2 * tid;
    const uint32_t c0 = b0 >= 0 ? sh.hist[b0] : 0, c1 = b1 >= 0 ? sh.hist[b1] : 0;
    uint64_t tot;
    const uint64_t incl = block_scan_incl(static_cast<uint64_t>(c0) + c1, sh, &tot);
    const uint64_t excl = incl - c0 - c1;
    if (b0 >= 0 && excl < remaining && excl + c0 >= remaining) {
      sh.sel_bin = static_cast<uint32_t>(b0);
      sh.sel_above = static_cast<uint32_t>(excl);
    }
    if (b1 >= 0 && excl + c0 < remaining && excl + c0 + c1 >= remaining) {
      sh.sel_bin = static_cast<uint32_t>(b1);
      sh.sel_above = static_cast<uint32_t>(excl + c0);
    }
    __syncthreads();
    prefix |= sh.sel_bin << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    remaining -= sh.sel_above;
    __syncthreads();
  }
  uint64_t bg = 0, be = 0;
  for (int64_t t0 = 0; t0 < nslots; t0 += kPart) {
    const int64_t i0 = t0 + static_cast<int64_t>(tid) * kItems;
    uint32_t keys[kItems];
    float v[kItems];
    int32_t ix[kItems];
    uint32_t vmask = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int64_t sl = i0 + j;
      const bool ok = slot_valid(sl);
      vmask |= static_cast<uint32_t>(ok) << j;
      v[j] = ok ? rv[sl] : 0.f;
      ix[j] = ok ? ri[sl] : 0;
      keys[j] = float_key(v[j]);
    }
    compact_tile(keys, vmask, prefix, remaining, sh, &bg, &be, [&](int j, uint64_t pos) {
      o[pos] = ix[j];
      if (os) os[pos] = v[j];
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
  hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a, np, cap,
                     cval, cidx, ccnt);
  return hipGetLastError();
}

}  // namespace csa
