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
struct Lds {
  static constexpr int KP = D + 8;  // K pitch (elements): 16-lane b128 reads hit distinct banks
  static constexpr int VP = D + 4;  // V pitch (elements): column reads of 4 row groups spread
  static constexpr int PP = kRows + 8;
  uint16_t k[kRows * KP];
  uint16_t v[kRows * VP];
  uint16_t p[kWaves][kHeadsPerWave * PP];
  int ok[kRows];
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_mfma(AttnArgs a, int sparse_i, int nsplit) {
  constexpr int KSQ = D / 32;  // k-steps of QK^T
  constexpr int NB = D / 16;   // 16-column output blocks
  constexpr int PIECES = D / 8;  // 16-byte pieces per row
  __shared__ Lds<D> sm;
  const bool sparse = sparse_i != 0;
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
  const RowMap rm = row_map(a, sparse, t);
  const int64_t n_rows = rm.n_cmp + rm.n_win;
  int64_t per = (n_rows + nsplit - 1) / nsplit;
  per = (per + kRows - 1) / kRows * kRows;
  const int64_t r_begin = split * per;
  const int64_t r_end = r_begin + per < n_rows ? r_begin + per : n_rows;

  const int h0 = static_cast<int>(hg * kHeadsPerWg + wave * kHeadsPerWave);
  // Q fragments (A operand): head h0 + c16, dims ks*32 + 8g .. +8.
  bf16x8 qf[KSQ];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (bt * a.H + h0 + c16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
  }
  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }
  const float sl2 = a.scale * kLog2e;

  const uint16_t* kcp = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vcp = static_cast<const uint16_t*>(a.vc);
  const uint16_t* krp = static_cast<const uint16_t*>(a.kr);
  const uint16_t* vrp = static_cast<const uint16_t*>(a.vr);

  for (int64_t c0 = r_begin; c0 < r_end; c0 += kRows) {
    // ---- stage 32 rows of K and V into LDS --------------------------------
    for (int id2 = threadIdx.x; id2 < kRows * PIECES; id2 += 256) {
      const int r = id2 / PIECES;
      const int p = id2 % PIECES;
      const int64_t v = c0 + r;
      bool raw = false;
      const int64_t off = v < r_end ? row_offset(a, sparse, rm, b, bt, v, &raw) : -1;
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (off >= 0) {
        const uint16_t* ks = raw ? krp : kcp;
        const uint16_t* vs = raw ? vrp : vcp;
        kk = *reinterpret_cast<const uint4*>(ks + off + p * 8);
        vv = *reinterpret_cast<const uint4*>(vs + off + p * 8);
      }
      *reinterpret_cast<uint4*>(&sm.k[r * Lds<D>::KP + p * 8]) = kk;
      uint2* vd = reinterpret_cast<uint2*>(&sm.v[r * Lds<D>::VP + p * 8]);
      vd[0] = make_uint2(vv.x, vv.y);
      vd[1] = make_uint2(vv.z, vv.w);
      if (p == 0) sm.ok[r] = off >= 0;
    }
    __syncthreads();

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
    // lane holds S[head 4g + r][row rb*16 + c16]
    const bool ok0 = sm.ok[c16] != 0, ok1 = sm.ok[16 + c16] != 0;
    float pv[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s0 = ok0 ? sacc[0][r] * sl2 : -INFINITY;
      const float s1 = ok1 ? sacc[1][r] * sl2 : -INFINITY;
      float cm = fmaxf(s0, s1);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
      const float mn = fmaxf(m_run[r], cm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m_run[r] - mu);
      pv[0][r] = fast_exp2(s0 - mu);
      pv[1][r] = fast_exp2(s1 - mu);
      l_run[r] = fmaf(l_run[r], alpha, pv[0][r] + pv[1][r]);
      m_run[r] = mn;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb][r] *= alpha;
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
    for (int nb = 0; nb < NB; ++nb) {
      bf16x8 vb;
      const uint16_t* vcol = &sm.v[(8 * g) * Lds<D>::VP + nb * 16 + c16];
#pragma unroll
      for (int e = 0; e < 8; ++e) vb[e] = __builtin_bit_cast(__bf16, vcol[e * Lds<D>::VP]);
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vb, oacc[nb], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------
  float l_tot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float s = l_run[r];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
    l_tot[r] = s;
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
      uint16_t* op = static_cast<uint16_t*>(a.out) + (bt * a.H + h) * D + c16;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) op[nb * 16] = f32_to_bf16(oacc[nb][r] * inv);
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
      for (int nb = 0; nb < NB; ++nb) wo[hl * D + nb * 16 + c16] = oacc[nb][r];
      if (c16 == 0) {
        wml[hl * 2 + 0] = m_run[r];
        wml[hl * 2 + 1] = l_tot[r];
      }
    }
  }
}

// Merge split partials: O = sum_s 2^{m_s-M} O_s / (sum_s 2^{m_s-M} l_s + 2^{sig-M}).
template <bool BF16>
__global__ __launch_bounds__(64) void attn_combine(AttnArgs a, int nsplit) {
  const int64_t bh = blockIdx.x;  // (bt, h)
  const int64_t bt = bh / a.H;
  const int64_t h = bh % a.H;
  const int64_t D = a.d;
  const float* wml = a.ws + static_cast<int64_t>(a.B * a.T) * nsplit * a.H * D;
  const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  float M = sig;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, wml[((bt * nsplit + s) * a.H + h) * 2]);
  float den = 0.f;
  if (M != -INFINITY) {
    den = sig == -INFINITY ? 0.f : fast_exp2(sig - M);
    for (int s = 0; s < nsplit; ++s) {
      const float ms = wml[((bt * nsplit + s) * a.H + h) * 2];
      if (ms != -INFINITY) den = fmaf(wml[((bt * nsplit + s) * a.H + h) * 2 + 1], fast_exp2(ms - M), den);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int64_t c = threadIdx.x; c < D; c += 64) {
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = wml[((bt * nsplit + s) * a.H + h) * 2];
      if (ms != -INFINITY) acc = fmaf(a.ws[((bt * nsplit + s) * a.H + h) * D + c], fast_exp2(ms - M), acc);
    }
    const float o = acc * inv;
    if (BF16)
      static_cast<uint16_t*>(a.out)[bh * D + c] = f32_to_bf16(o);
    else
      static_cast<float*>(a.out)[bh * D + c] = o;
  }
  if (a.lse && threadIdx.x == 0) a.lse[bh] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
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
  const int64_t target = 512;  // two resident workgroups on each of 256 CUs
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
  switch (a.d) {
    case 128: hipLaunchKernelGGL(attn_mfma<128>, grid, dim3(256), 0, s, a, sparse ? 1 : 0, nsplit); break;
    case 256: hipLaunchKernelGGL(attn_mfma<256>, grid, dim3(256), 0, s, a, sparse ? 1 : 0, nsplit); break;
    case 512: hipLaunchKernelGGL(attn_mfma<512>, grid, dim3(256), 0, s, a, sparse ? 1 : 0, nsplit); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(attn_combine<true>, dim3(static_cast<uint32_t>(a.B * a.T * a.H)), dim3(64), 0, s, a,
                     nsplit);
  return hipGetLastError();
}

bool attn_shape_supported(int64_t H, int64_t d, bool bf16) {
  if (!bf16) return d >= 1 && d <= 512;
  return H % kHeadsPerWg == 0 && (d == 128 || d == 256 || d == 512);
}

}  // namespace csa
