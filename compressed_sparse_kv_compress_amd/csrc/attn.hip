// MQA attention with an attention sink over a per-query list of rows.
//
//   CSA (sparse): rows = the top-k selected compressed entries (idx, -1 =
//                 empty slot) followed by the raw window tokens
//                 max(0, t-W+1) .. t.
//   HCA (dense):  rows = every visible compressed entry [0, floor(t/m))
//                 followed by the same optional raw window.
//
// out[t][h] = sum_i p_i v_i,  p_i = e^{l_i} / (e^{sigma_h} + sum_j e^{l_j}),
// l_i = scale * q[t][h] . k_i;  lse = log(e^{sigma_h} + sum_j e^{l_j}).
//
// Method: shareware.cn Hybrid Attention article, sections 三.1 (128 raw
// tokens), 八 (HCA reads every entry densely), 十 (the window covers the
// same-block history that compressed entries cannot), 十一 (MQA: all query
// heads share one K/V) and 十二 (a sink logit with no value); trdm.cn
// attention article, section 3.1 (online softmax with running max and sum)
// and 4.3 (compressed rows concatenated with the uncompressed window).
//
// Design (gfx950, bf16): 64 query heads share every K/V row, so QK^T and PV
// are dense contractions with the heads as the M dimension: MFMA
// v_mfma_f32_16x16x32_bf16, one wavefront per 16 heads, four wavefronts
// (64 heads) per workgroup.  Rows are staged 32 at a time into LDS (K and V
// row-major, padded pitches so the MFMA operand reads are bank-conflict
// free), gathered through the index list for CSA or streamed contiguously for
// HCA; one staged row serves all 64 heads.  The softmax is online in log2
// units, P goes back through a small per-wave LDS tile to MFMA A layout, and
// the 16 heads x d output accumulators live in VGPRs (d = 512: 128 per lane).
// Decode queries are split over the row list (flash-decoding) and merged by a
// log-sum-exp combine kernel that also applies the sink; prefill-sized launches
// use one workgroup per (query, 64 heads) and finish in place.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {
namespace {

constexpr int kRows = 32;  // rows staged per chunk
constexpr int kHeadsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kHeadsPerWg = kHeadsPerWave * kWaves;

struct RowMap {
  int64_t n_cmp;   // compressed slots (sparse: k, dense: visible count)
  int64_t n_win;   // window rows
  int64_t win_lo;  // first raw position of the window
};

__device__ __forceinline__ RowMap row_map(const AttnArgs& a, bool sparse, int64_t t) {
  RowMap r;
  if (sparse) {
    r.n_cmp = a.k;
  } else {
    int64_t nv = t / a.m;
    r.n_cmp = nv < a.L ? nv : a.L;
  }
  if (a.W > 0) {
    int64_t lo = t - a.W + 1;
    if (lo < 0) lo = 0;
    r.win_lo = lo;
    r.n_win = t - lo + 1;
  } else {
    r.win_lo = 0;
    r.n_win = 0;
  }
  return r;
}

// Element offset of virtual row v of query (b, bt) in its source, or -1 if the
// row is empty.  *from_raw tells which source (compressed cache or window).
__device__ __forceinline__ int64_t row_offset(const AttnArgs& a, bool sparse, const RowMap& rm,
                                              int64_t b, int64_t bt, int64_t v, bool* from_raw) {
  if (v < rm.n_cmp) {
    *from_raw = false;
    int64_t s = v;
    if (sparse) {
      s = a.idx[bt * a.k + v];
      if (s < 0 || s >= a.L) return -1;
    }
    return (b * a.L + s) * a.d;
  }
  const int64_t w = v - rm.n_cmp;
  if (w >= rm.n_win) return -1;
  *from_raw = true;
  const int64_t u = rm.win_lo + w - (a.n_ctx - a.R);
  return (b * a.R + u) * a.d;
}

template <int D>
struct __attribute__((aligned(16))) Lds {
  static constexpr int KP = D + 8;  // row pitch (elements) of staged K and V rows
  static constexpr int PP = kRows + 8;
  uint16_t k[kRows * KP];
  uint16_t v[kRows * KP];
  uint16_t p[kWaves][kHeadsPerWave * PP];
  int ok[kRows];
};

// Output-column layout of PV: dims are taken in slabs of 128; inside a slab,
// lane column c (0..15) of N-block e (0..7) is dim 8c + e.  A lane then reads
// 8 consecutive dims of a staged V row with one 16-byte LDS load and
// transposes 8 such rows in registers into the 8 B operands of the slab.
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);  // (x.lo, y.lo)
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);  // (x.hi, y.hi)
}

template <int D, bool SPARSE>
__global__ __launch_bounds__(256, 1) void attn_mfma(AttnArgs a, int nsplit) {
  constexpr int KSQ = D / 32;    // k-steps of QK^T
  constexpr int NB = D / 16;     // 16-column output blocks
  constexpr int SLABS = D / 128;
  constexpr int PIECES = D / 8;  // 16-byte pieces per row
  constexpr int PER = kRows * PIECES / 256;  // pieces per thread per chunk
  constexpr float kRebase = 8.f;  // re-base the running max only when it grows by > 2^8
  __shared__ Lds<D> sm;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;     // 16-lane group
  const int c16 = lane & 15;

  const int64_t hgroups = a.H / kHeadsPerWg;
  int64_t id = blockIdx.x;
  const int split = static_cast<int>(id % nsplit);
  id /= nsplit;
  const int64_t hg = id % hgroups;
  const int64_t bt = id / hgroups;
  const int64_t b = bt / a.T;
  const int64_t t = a.n_ctx - a.T + bt % a.T;
  const RowMap rm = row_map(a, SPARSE, t);
  const int64_t n_rows = rm.n_cmp + rm.n_win;
  int64_t per = (n_rows + nsplit - 1) / nsplit;
  per = (per + kRows - 1) / kRows * kRows;
  const int64_t r_begin = split * per;
  const int64_t r_end = r_begin + per < n_rows ? r_begin + per : n_rows;

  // Register staging of one 32-row chunk: every global load of the chunk is
  // issued back to back with no control flow around it (an empty row loads
  // from a valid dummy address and is zeroed afterwards); the chunk after the
  // current one is in flight while the current one is being computed.
  const uint16_t* dummy = static_cast<const uint16_t*>(a.q) + bt * a.H * D;
  const uint16_t* kcb = static_cast<const uint16_t*>(a.kc) + b * a.L * D;
  const uint16_t* vcb = static_cast<const uint16_t*>(a.vc) + b * a.L * D;
  const uint16_t* krb = static_cast<const uint16_t*>(a.kr) + b * a.R * D;
  const uint16_t* vrb = static_cast<const uint16_t*>(a.vr) + b * a.R * D;
  const int64_t win0 = rm.win_lo - (a.n_ctx - a.R) - rm.n_cmp;  // raw row of virtual row v is v + win0
  const int pc = threadIdx.x % PIECES;
  const int r0 = threadIdx.x / PIECES;
  u32x4 kp[PER], vp[PER];
  uint32_t okmask = 0;
  auto issue = [&](int64_t c0) {
    int32_t sid[PER];
    if (SPARSE && a.k > 0) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int64_t v = c0 + r0 + (256 / PIECES) * i;
        v = v < a.k - 1 ? v : a.k - 1;
        sid[i] = a.idx[bt * a.k + v];
      }
    }
    okmask = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t v = c0 + r0 + (256 / PIECES) * i;
      const bool cmp = v < rm.n_cmp;
      const int64_t s = SPARSE ? (a.k > 0 ? static_cast<int64_t>(sid[i]) : -1) : v;
      const bool ok = v < r_end && (cmp ? (!SPARSE || (s >= 0 && s < a.L)) : true);
      const int64_t off = (cmp ? s : v + win0) * D + pc * 8;
      const uint16_t* kb = ok ? (cmp ? kcb : krb) + off : dummy + pc * 8;
      const uint16_t* vb = ok ? (cmp ? vcb : vrb) + off : dummy + pc * 8;
      kp[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb));
      vp[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb));
      okmask |= static_cast<uint32_t>(ok) << i;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = r0 + (256 / PIECES) * i;
      const bool ok = (okmask >> i) & 1u;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&sm.k[r * Lds<D>::KP + pc * 8]) = ok ? kp[i] : z;
      *reinterpret_cast<u32x4*>(&sm.v[r * Lds<D>::KP + pc * 8]) = ok ? vp[i] : z;
      if (pc == 0) sm.ok[r] = ok;
    }
  };
  // Q is loaded before the first chunk so that the chunk's wait also covers it
  // (otherwise the wait counter can not prove Q complete inside the loop and
  // every chunk would wait for its own prefetch).
  const int h0 = static_cast<int>(hg * kHeadsPerWg + wave * kHeadsPerWave);
  // Q fragments (A operand): head h0 + c16, dims ks*32 + 8g .. +8.
  bf16x8 qf[KSQ];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (bt * a.H + h0 + c16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
  }
  if (r_begin < r_end) issue(r_begin);

  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }
  const float sl2 = a.scale * kLog2e;

  for (int64_t c0 = r_begin; c0 < r_end; c0 += kRows) {
    stash();
    __syncthreads();
    if (c0 + kRows < r_end) issue(c0 + kRows);

    // ---- S = Q K^T for 16 heads x 32 rows ---------------------------------
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 kb =
            *reinterpret_cast<const bf16x8*>(&sm.k[(rb * 16 + c16) * Lds<D>::KP + ks * 32 + 8 * g]);
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kb, sacc[rb], 0, 0, 0);
      }
    // lane holds S[head 4g + r][row rb*16 + c16]; online softmax in log2
    // units against a lazily re-based running max.
    const bool ok0 = sm.ok[c16] != 0, ok1 = sm.ok[16 + c16] != 0;
    float s0[4], s1[4], mnew[4];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s0[r] = ok0 ? sacc[0][r] * sl2 : -INFINITY;
      s1[r] = ok1 ? sacc[1][r] * sl2 : -INFINITY;
      float cm = fmaxf(s0[r], s1[r]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
      mnew[r] = fmaxf(m_run[r], cm);
      grow |= m_run[r] != -INFINITY && mnew[r] > m_run[r] + kRebase;
    }
    if (__any(grow)) {  // rare: re-base output and sums to the new max
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float alpha = m_run[r] == -INFINITY ? 1.f : fast_exp2(m_run[r] - mnew[r]);
        l_run[r] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][r] *= alpha;
        m_run[r] = mnew[r];
      }
    }
    float pv[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (m_run[r] == -INFINITY) m_run[r] = mnew[r];  // first rows of this head: nothing to re-base
      const float mu = m_run[r] == -INFINITY ? 0.f : m_run[r];
      pv[0][r] = fast_exp2(s0[r] - mu);
      pv[1][r] = fast_exp2(s1[r] - mu);
      l_run[r] += pv[0][r] + pv[1][r];
    }
    // P (bf16) to LDS as [head][row] for the A operand of PV.
    uint16_t* pw = sm.p[wave];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[(4 * g + r) * Lds<D>::PP + rb * 16 + c16] = f32_to_bf16(pv[rb][r]);
    __syncthreads();

    // ---- O += P V -----------------------------------------------------------
    const bf16x8 pf = *reinterpret_cast<const bf16x8*>(&pw[c16 * Lds<D>::PP + 8 * g]);
#pragma unroll
    for (int sb = 0; sb < SLABS; ++sb) {
      u32x4 rowv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        rowv[j] = *reinterpret_cast<const u32x4*>(&sm.v[(8 * g + j) * Lds<D>::KP + sb * 128 + 8 * c16]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 ev, od;  // dims 8c16 + 2w (even) and + 2w+1 (odd), rows 8g .. 8g+7
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ev[u] = lo_pair(rowv[2 * u][w], rowv[2 * u + 1][w]);
          od[u] = hi_pair(rowv[2 * u][w], rowv[2 * u + 1][w]);
        }
        oacc[sb * 8 + 2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pf, __builtin_bit_cast(bf16x8, ev), oacc[sb * 8 + 2 * w], 0, 0, 0);
        oacc[sb * 8 + 2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pf, __builtin_bit_cast(bf16x8, od), oacc[sb * 8 + 2 * w + 1], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: oacc[sb*8 + e][r] = O[head 4g+r][dim sb*128 + 8*c16 + e] ----
  float l_tot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float sum = l_run[r];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
    l_tot[r] = sum;
  }
  if (nsplit == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = h0 + 4 * g + r;
      const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(m_run[r], sig);
      float den = 0.f, f = 0.f;
      if (M != -INFINITY) {
        f = m_run[r] == -INFINITY ? 0.f : fast_exp2(m_run[r] - M);
        den = l_tot[r] * f + (sig == -INFINITY ? 0.f : fast_exp2(sig - M));
      }
      const float inv = den > 0.f ? f / den : 0.f;
      uint16_t* op = static_cast<uint16_t*>(a.out) + (bt * a.H + h) * D + 8 * c16;
#pragma unroll
      for (int sb = 0; sb < SLABS; ++sb) {
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          w[u] = pack_bf16x2(oacc[sb * 8 + 2 * u][r] * inv, oacc[sb * 8 + 2 * u + 1][r] * inv);
        *reinterpret_cast<u32x4*>(op + sb * 128) = w;
      }
      if (a.lse && c16 == 0) a.lse[bt * a.H + h] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
    }
  } else {
    float* wo = a.ws + ((bt * nsplit + split) * a.H + h0) * D;
    float* wml = a.ws + static_cast<int64_t>(a.B * a.T) * nsplit * a.H * D +
                 ((bt * nsplit + split) * a.H + h0) * 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hl = 4 * g + r;
#pragma unroll
      for (int sb = 0; sb < SLABS; ++sb) {
        f32x4 lo = f32x4{oacc[sb * 8 + 0][r], oacc[sb * 8 + 1][r], oacc[sb * 8 + 2][r], oacc[sb * 8 + 3][r]};
        f32x4 hi = f32x4{oacc[sb * 8 + 4][r], oacc[sb * 8 + 5][r], oacc[sb * 8 + 6][r], oacc[sb * 8 + 7][r]};
        float* dst = wo + hl * D + sb * 128 + 8 * c16;
        *reinterpret_cast<f32x4*>(dst) = lo;
        *reinterpret_cast<f32x4*>(dst + 4) = hi;
      }
      if (c16 == 0) {
        wml[hl * 2 + 0] = m_run[r];
        wml[hl * 2 + 1] = l_tot[r];
      }
    }
  }
}

// Merge split partials: O = sum_s 2^{m_s-M} O_s / (sum_s 2^{m_s-M} l_s + 2^{sig-M}).
// One 256-thread workgroup per (query, head): the split weights go to LDS
// once, then every thread merges two adjacent output dims across the splits.
template <bool BF16>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int nsplit) {
  __shared__ float fac[64];
  __shared__ float inv_sh, lse_sh;
  const int64_t bh = blockIdx.x;  // (bt, h)
  const int64_t bt = bh / a.H;
  const int64_t h = bh % a.H;
  const int64_t D = a.d;
  const float* wml = a.ws + static_cast<int64_t>(a.B * a.T) * nsplit * a.H * D;
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float ms = s < nsplit ? wml[((bt * nsplit + s) * a.H + h) * 2] : -INFINITY;
    const float ls = s < nsplit ? wml[((bt * nsplit + s) * a.H + h) * 2 + 1] : 0.f;
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float M = fmaxf(wave_max(ms), sig);
    const float f = (M == -INFINITY || ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
    fac[s] = f;
    float den = wave_sum(ls * f);
    if (M != -INFINITY && sig != -INFINITY) den += fast_exp2(sig - M);
    if (s == 0) {
      inv_sh = den > 0.f ? 1.f / den : 0.f;
      lse_sh = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  const float inv = inv_sh;
  for (int64_t c = 2 * threadIdx.x; c < D; c += 512) {
    float a0 = 0.f, a1 = 0.f;
    const float* src = a.ws + (bt * nsplit * a.H + h) * D + c;
    for (int s = 0; s < nsplit; ++s) {
      const float2 v = *reinterpret_cast<const float2*>(src + static_cast<int64_t>(s) * a.H * D);
      a0 = fmaf(v.x, fac[s], a0);
      a1 = fmaf(v.y, fac[s], a1);
    }
    if (BF16) {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + bh * D + c) = pack_bf16x2(a0 * inv, a1 * inv);
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + bh * D + c) = make_float2(a0 * inv, a1 * inv);
    }
  }
  if (a.lse && threadIdx.x == 0) a.lse[bh] = lse_sh;
}

// fp32 storage: one wavefront per (query, head), VALU, 64 rows per step.
__global__ __launch_bounds__(64) void attn_f32(AttnArgs a, int sparse_i) {
  extern __shared__ float qs[];
  __shared__ int64_t voff[64];
  __shared__ int vraw[64];
  __shared__ float pbuf[64];
  const bool sparse = sparse_i != 0;
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t bt = bh / a.H;
  const int64_t h = bh % a.H;
  const int64_t b = bt / a.T;
  const int64_t t = a.n_ctx - a.T + bt % a.T;
  const int64_t D = a.d;
  const float* q = static_cast<const float*>(a.q) + bh * D;
  for (int64_t c = lane; c < D; c += 64) qs[c] = q[c];
  __syncthreads();
  const RowMap rm = row_map(a, sparse, t);
  const int64_t n_rows = rm.n_cmp + rm.n_win;
  const float sl2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  const float* kcp = static_cast<const float*>(a.kc);
  const float* vcp = static_cast<const float*>(a.vc);
  const float* krp = static_cast<const float*>(a.kr);
  const float* vrp = static_cast<const float*>(a.vr);
  for (int64_t c0 = 0; c0 < n_rows; c0 += 64) {
    const int64_t v = c0 + lane;
    bool raw = false;
    const int64_t off = v < n_rows ? row_offset(a, sparse, rm, b, bt, v, &raw) : -1;
    float lg = -INFINITY;
    if (off >= 0) {
      const float* kp = (raw ? krp : kcp) + off;
      float dot = 0.f;
      for (int64_t c = 0; c < D; ++c) dot = fmaf(qs[c], kp[c], dot);
      lg = dot * sl2;
    }
    const float mn = fmaxf(m_run, wave_max(lg));
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m_run - mu);
    const float p = fast_exp2(lg - mu);
    l_run = fmaf(l_run, alpha, wave_sum(p));
    m_run = mn;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    voff[lane] = off;
    vraw[lane] = raw;
    pbuf[lane] = p;
    __syncthreads();
    for (int j = 0; j < 64; ++j) {
      const int64_t vo = voff[j];
      if (vo < 0) continue;
      const float pj = pbuf[j];
      const float* vp = (vraw[j] ? vrp : vcp) + vo;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (lane + 64 * i < D) o[i] = fmaf(pj, vp[lane + 64 * i], o[i]);
    }
    __syncthreads();
  }
  const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  const float M = fmaxf(m_run, sig);
  float den = 0.f, f = 0.f;
  if (M != -INFINITY) {
    f = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
    den = l_run * f + (sig == -INFINITY ? 0.f : fast_exp2(sig - M));
  }
  const float inv = den > 0.f ? f / den : 0.f;
  float* op = static_cast<float*>(a.out) + bh * D;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (lane + 64 * i < D) op[lane + 64 * i] = o[i] * inv;
  if (a.lse && lane == 0) a.lse[bh] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace

int attn_splits(int64_t B, int64_t T, int64_t H, int64_t d, int64_t max_rows, bool bf16) {
  (void)d;
  if (!bf16) return 1;
  const int64_t base = B * T * (H / kHeadsPerWg);
#ifndef CSA_ATTN_TARGET
#define CSA_ATTN_TARGET 256
#endif
  const int64_t target = CSA_ATTN_TARGET;  // workgroups wanted per launch (one per CU)
  int64_t ns = (target + base - 1) / base;
  const int64_t cap = (max_rows + 63) / 64;  // keep >= 64 rows per split
  if (ns > cap) ns = cap;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  return static_cast<int>(ns);
}

size_t attn_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t d, int nsplit) {
  if (nsplit <= 1) return 0;
  return static_cast<size_t>(B * T) * nsplit * H * (d + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a, bool sparse, bool bf16, int nsplit, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  if (!bf16) {
    hipLaunchKernelGGL(attn_f32, dim3(static_cast<uint32_t>(a.B * a.T * a.H)), dim3(64),
                       a.d * sizeof(float), s, a, sparse ? 1 : 0);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<uint32_t>(a.B * a.T * (a.H / kHeadsPerWg) * nsplit));
#define CSA_ATTN_LAUNCH(D_)                                                                            \
  case D_:                                                                                             \
    if (sparse) hipLaunchKernelGGL((attn_mfma<D_, true>), grid, dim3(256), 0, s, a, nsplit);           \
    else hipLaunchKernelGGL((attn_mfma<D_, false>), grid, dim3(256), 0, s, a, nsplit);                 \
    break;
  switch (a.d) {
    CSA_ATTN_LAUNCH(128)
    CSA_ATTN_LAUNCH(256)
    CSA_ATTN_LAUNCH(512)
    default: return hipErrorInvalidValue;
  }
#undef CSA_ATTN_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(attn_combine<true>, dim3(static_cast<uint32_t>(a.B * a.T * a.H)), dim3(256), 0, s, a,
                     nsplit);
  return hipGetLastError();
}

bool attn_shape_supported(int64_t H, int64_t d, bool bf16) {
  if (!bf16) return d >= 1 && d <= 512;
  return H % kHeadsPerWg == 0 && (d == 128 || d == 256 || d == 512);
}

}  // namespace csa
