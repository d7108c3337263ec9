// Top-k selection over indexer scores: per query keep the min(k, |V_t|)
// highest scores among the visible entries, equal scores going to the lower
// entry index; write the kept indices in ascending order, -1 padded.
//
// Method: shareware.cn Hybrid Attention article, section 六 (score the
// compressed entries, keep the top-k candidates for the main attention);
// aimodeling.com news item, CSA paragraph (1024 entries per query).
//
// Design (gfx950): exact radix select on order-preserving 32-bit keys
// (-0 and +0 share a key, so they tie).  One 1024-thread workgroup per query
// row: three histogram passes of 11, 11 and 10 bits in LDS pin down the key
// of the k-th largest score and how many entries equal to it are taken.  A
// final pass walks the row in index order in 8192-entry tiles; a single
// 64-bit block scan per tile (count of strictly-greater entries in the low
// word, count of threshold-equal entries in the high word) gives every kept
// entry its output slot, so the output comes out sorted by index without a
// sort and the lower-index tie rule is exact.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 8;

// Inclusive scan of one 64-bit value per thread across the workgroup.
// Returns the inclusive prefix; *total receives the workgroup sum.
__device__ __forceinline__ uint64_t block_scan_incl(uint64_t v, uint64_t* sh, uint64_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint64_t w = lane < kWaves ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const uint64_t y = __shfl_up(w, o, 64);
      if (lane >= o) w += y;
    }
    if (lane < kWaves) sh[kWaves + lane] = w;
  }
  __syncthreads();
  const uint64_t before = wave ? sh[kWaves + wave - 1] : 0;
  *total = sh[2 * kWaves - 1];
  __syncthreads();
  return v + before;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint64_t scan_sh[2 * kWaves];
  __shared__ uint32_t sel_bin, sel_above;

  const int64_t lrow = blockIdx.x;
  const int64_t row = a.row0 + lrow;
  const int64_t tpos = a.n_ctx - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  if (nv < 0) nv = 0;
  const float* s = a.score + lrow * a.ld;
  int32_t* o = a.idx + lrow * a.k;
  float* os = a.out_score ? a.out_score + lrow * a.k : nullptr;
  const int tid = threadIdx.x;

  if (nv <= a.k) {
    for (int64_t i = tid; i < a.k; i += kThreads) {
      o[i] = i < nv ? static_cast<int32_t>(i) : -1;
      if (os) os[i] = i < nv ? s[i] : -INFINITY;
    }
    return;
  }

  // ---- radix select of the k-th largest key -------------------------------
  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(a.k);
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    for (int i = tid; i < 2048; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < nv; i += kThreads) {
      const uint32_t key = float_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // Scan bins from the top: thread i owns bins nb-1-2i and nb-2-2i.
    const int b0 = nb - 1 - 2 * tid, b1 = nb - 2 - 2 * tid;
    const uint32_t c0 = b0 >= 0 ? hist[b0] : 0, c1 = b1 >= 0 ? hist[b1] : 0;
    uint64_t tot;
    const uint64_t incl = block_scan_incl(static_cast<uint64_t>(c0) + c1, scan_sh, &tot);
    const uint64_t excl = incl - c0 - c1;
    if (b0 >= 0 && excl < remaining && excl + c0 >= remaining) {
      sel_bin = static_cast<uint32_t>(b0);
      sel_above = static_cast<uint32_t>(excl);
    }
    if (b1 >= 0 && excl + c0 < remaining && excl + c0 + c1 >= remaining) {
      sel_bin = static_cast<uint32_t>(b1);
      sel_above = static_cast<uint32_t>(excl + c0);
    }
    __syncthreads();
    prefix |= sel_bin << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
    remaining -= sel_above;
    __syncthreads();
  }
  const uint32_t thr = prefix;         // key of the k-th largest score
  const uint64_t take_eq = remaining;  // entries equal to it that are kept

  // ---- ordered compaction -------------------------------------------------
  uint64_t base_gt = 0, base_eq = 0;
  for (int64_t t0 = 0; t0 < nv; t0 += static_cast<int64_t>(kThreads) * kItems) {
    const int64_t i0 = t0 + static_cast<int64_t>(tid) * kItems;
    uint32_t keys[kItems];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      keys[j] = (i0 + j < nv) ? float_key(s[i0 + j]) : 0u;
      ngt += (i0 + j < nv) && keys[j] > thr;
      neq += (i0 + j < nv) && keys[j] == thr;
    }
    uint64_t tot;
    const uint64_t packed = (static_cast<uint64_t>(neq) << 32) | ngt;
    const uint64_t excl = block_scan_incl(packed, scan_sh, &tot) - packed;
    uint64_t gt_before = base_gt + (excl & 0xffffffffu);
    uint64_t eq_before = base_eq + (excl >> 32);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      if (i0 + j >= nv) break;
      const bool gt = keys[j] > thr;
      const bool eq = keys[j] == thr;
      if (gt || (eq && eq_before < take_eq)) {
        const uint64_t pos = gt_before + (eq_before < take_eq ? eq_before : take_eq);
        o[pos] = static_cast<int32_t>(i0 + j);
        if (os) os[pos] = s[i0 + j];
      }
      gt_before += gt;
      eq_before += eq;
    }
    base_gt += tot & 0xffffffffu;
    base_eq += tot >> 32;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.nrows == 0 || a.k == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<uint32_t>(a.nrows)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
