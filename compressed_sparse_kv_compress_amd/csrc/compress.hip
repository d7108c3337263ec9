// Block-weighted compression: one compressed entry per block of m raw tokens.
//
// Method: shareware.cn Hybrid Attention article, section 四 (per-dimension,
// token-dependent softmax weights instead of a plain mean) and section 五
// (two-path overlap: the current block through stream A, the previous block
// through stream B, one joint softmax per channel); trdm.cn attention
// article, section 4.3 改进二 (two streams with their own position biases).
//
// Design (gfx950): a pure HBM stream at ~2 flop per byte.  One thread owns
// 16 bytes of channels (8 bf16 or 4 fp32) of one entry, so a wavefront reads
// 1 KiB contiguous per raw row (fully coalesced 16-byte loads).  Candidates are
// taken 8 tokens at a time: all 8 logit/value loads are issued before any use
// (memory-level parallelism), the chunk maximum is formed in registers and the
// running sums are rescaled once per chunk, so there is about one exp2 per
// element.  Weights are never materialised.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kChunk = 8;

template <Dt DT>
struct Io;

template <>
struct Io<kBF16> {
  static constexpr int VEC = 8;
  __device__ static void load(const void* base, int64_t off, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    v[0] = lo_bf16(w.x); v[1] = hi_bf16(w.x);
    v[2] = lo_bf16(w.y); v[3] = hi_bf16(w.y);
    v[4] = lo_bf16(w.z); v[5] = hi_bf16(w.z);
    v[6] = lo_bf16(w.w); v[7] = hi_bf16(w.w);
  }
  __device__ static void store(void* base, int64_t off, const float* v) {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = w;
  }
};

// FP8 (OCP E4M3): 8 channels (8 bytes) per thread; the hardware converters
// decode exactly and encode with round-to-nearest-even.
template <>
struct Io<kFP8> {
  static constexpr int VEC = 8;
  __device__ static void load(const void* base, int64_t off, float* v) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + off);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int word = static_cast<int>(h ? w.y : w.x);
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      v[4 * h + 0] = lo[0];
      v[4 * h + 1] = lo[1];
      v[4 * h + 2] = hi[0];
      v[4 * h + 3] = hi[1];
    }
  }
  __device__ static void store(void* base, int64_t off, const float* v) {
    uint2 w;
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], x, true);
    int y = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    y = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], y, true);
    w.x = static_cast<uint32_t>(x);
    w.y = static_cast<uint32_t>(y);
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + off) = w;
  }
};

template <>
struct Io<kF32> {
  static constexpr int VEC = 4;
  __device__ static void load(const void* base, int64_t off, float* v) {
    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
  __device__ static void store(void* base, int64_t off, const float* v) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// The candidates of entry j form one virtual list: stream-B tokens
// (j-1)*m .. j*m-1 first (two-path, j >= 1), then stream-A tokens
// j*m .. min((j+1)*m, n)-1.  Candidate i maps to its stream, raw row and
// bias row here.
struct Cands {
  int64_t nb, na, b_lo, a_lo, a_bias0;
};

// Fold candidates [lo, hi) of the virtual list into the running (max,
// denominator, numerator) of VEC channels.  Logits are in log2 units.
template <Dt DT>
__device__ __forceinline__ void fold_range(const CompressArgs& a, const Cands& cd, int64_t lo, int64_t hi,
                                           int64_t row_base, int64_t c0, float* mx, float* den, float* acc) {
  constexpr int VEC = Io<DT>::VEC;
  for (int64_t i0 = lo; i0 < hi; i0 += kChunk) {
    // All 2 x kChunk loads are issued unconditionally (candidates past the
    // end re-read the last one and are masked below), so they are all in
    // flight together instead of being serialised by control flow.
    float xv[kChunk][VEC], lv[kChunk][VEC];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int64_t ci = i0 + i < hi ? i0 + i : hi - 1;
      const bool from_b = ci < cd.nb;
      const int64_t u = from_b ? cd.b_lo + ci : cd.a_lo + (ci - cd.nb);
      const int64_t off = (row_base + (u - a.p0)) * a.D + c0;
      Io<DT>::load(from_b ? a.x_b : a.x_a, off, xv[i]);
      Io<DT>::load(from_b ? a.z_b : a.z_a, off, lv[i]);
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const bool ok = i0 + i < hi;
      if (a.bias) {
        const int64_t ci = ok ? i0 + i : hi - 1;
        const int64_t brow = ci < cd.nb ? ci : cd.a_bias0 + (ci - cd.nb);
        const float* br = a.bias + brow * a.D + c0;
#pragma unroll
        for (int c = 0; c < VEC; ++c) lv[i][c] += br[c];
      }
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        lv[i][c] = ok ? lv[i][c] * kLog2e : -INFINITY;
        xv[i][c] = ok ? xv[i][c] : 0.f;
      }
    }
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      float cm = lv[0][c];
#pragma unroll
      for (int i = 1; i < kChunk; ++i) cm = fmaxf(cm, lv[i][c]);
      const float nm = fmaxf(mx[c], cm);
      if (nm == -INFINITY) continue;  // nothing finite yet in this channel
      const float f = fast_exp2(mx[c] - nm);
      float sd = 0.f, sa = 0.f;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const float e = fast_exp2(lv[i][c] - nm);
        sd += e;
        sa = fmaf(e, xv[i][c], sa);
      }
      den[c] = fmaf(den[c], f, sd);
      acc[c] = fmaf(acc[c], f, sa);
      mx[c] = nm;
    }
  }
}

// S = 1: one thread per (entry, 16-byte channel group), for bulk launches.
// S > 1: the candidate tokens of each segment are split over S thread slices,
// S consecutive lanes of one wavefront, whose partial (max, denominator,
// numerator) are merged with lane exchanges; used when a launch has too few
// entries to fill the GPU (decode-time refresh).  The kernel uses no LDS, so
// its workgroups can share a CU with an LDS-heavy kernel running beside it
// (the indexer scan holds almost all of a CU's LDS).
template <Dt DT, int S>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  static_assert(S >= 1 && S <= 64 && (S & (S - 1)) == 0, "slices: a power of two within a wavefront");
  constexpr int VEC = Io<DT>::VEC;
  constexpr int LANES = 256 / S;  // channel groups per workgroup
  const int slice = threadIdx.x % S;
  const int lane = threadIdx.x / S;
  const int64_t nvec = a.D / VEC;
  const int64_t ne = a.e1 - a.e0;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * LANES + lane;
  const bool live = gid < a.B * ne * nvec;
  const int64_t g = live ? gid : 0;
  const int64_t cv = g % nvec;
  const int64_t tmp = g / nvec;
  const int64_t jj = tmp % ne;
  const int64_t b = tmp / ne;
  const int64_t j = a.e0 + jj;
  const int64_t c0 = cv * VEC;
  const int64_t row_base = b * a.n_raw;

  float mx[VEC], den[VEC], acc[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) { mx[c] = -INFINITY; den[c] = 0.f; acc[c] = 0.f; }

  const bool two = a.x_b != nullptr;
  Cands cd;
  cd.nb = (two && j >= 1) ? a.m : 0;
  cd.b_lo = (j - 1) * a.m;
  cd.a_lo = j * a.m;
  cd.na = ((j + 1) * a.m < a.n ? (j + 1) * a.m : a.n) - cd.a_lo;
  cd.a_bias0 = two ? a.m : 0;
  const int64_t total = cd.nb + cd.na;
  int64_t lo = 0, hi = total;
  if (S > 1) {
    const int64_t per = (total + S - 1) / S;
    lo = slice * per;
    hi = lo + per < total ? lo + per : total;
  }
  if (live && lo < hi) fold_range<DT>(a, cd, lo, hi, row_base, c0, mx, den, acc);

  if (S > 1) {
    // Pairwise merges over the S lanes (xor distance 1, 2, ...): both lanes
    // of a pair evaluate the same expression with the lower lane's partial
    // first, so they agree bit for bit.
#pragma unroll
    for (int off = 1; off < S; off <<= 1) {
      const bool low = (slice & off) == 0;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const float m2 = __shfl_xor(mx[c], off, 64);
        const float d2 = __shfl_xor(den[c], off, 64);
        const float a2 = __shfl_xor(acc[c], off, 64);
        const float ml = low ? mx[c] : m2, mh = low ? m2 : mx[c];
        const float dl = low ? den[c] : d2, dh = low ? d2 : den[c];
        const float al = low ? acc[c] : a2, ah = low ? a2 : acc[c];
        const float M = fmaxf(ml, mh);
        const float fl = ml == -INFINITY ? 0.f : fast_exp2(ml - M);
        const float fh = mh == -INFINITY ? 0.f : fast_exp2(mh - M);
        mx[c] = M;
        den[c] = fmaf(dl, fl, dh * fh);
        acc[c] = fmaf(al, fl, ah * fh);
      }
    }
    if (slice != 0) return;
  }
  if (!live) return;
  float o[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) o[c] = den[c] > 0.f ? acc[c] / den[c] : 0.f;
  Io<DT>::store(a.out, (b * a.out_ld + jj) * a.D + c0, o);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, Dt dt, hipStream_t s) {
  const int vec = dt == kF32 ? 4 : 8;
  const int64_t total = a.B * (a.e1 - a.e0) * (a.D / vec);
  if (total == 0) return hipSuccess;
  // Few entries with long blocks: spread each block's tokens over 16 slices.
  const bool sliced = total < 32768 && a.m >= 32;
  const dim3 grid(static_cast<uint32_t>(sliced ? (total + 15) / 16 : (total + 255) / 256));
#define CSA_COMPRESS_LAUNCH(DT_)                                                          \
  if (sliced) hipLaunchKernelGGL((compress_kernel<DT_, 16>), grid, dim3(256), 0, s, a);  \
  else hipLaunchKernelGGL((compress_kernel<DT_, 1>), grid, dim3(256), 0, s, a);
  switch (dt) {
    case kBF16: CSA_COMPRESS_LAUNCH(kBF16) break;
    case kFP8: CSA_COMPRESS_LAUNCH(kFP8) break;
    default: CSA_COMPRESS_LAUNCH(kF32) break;
  }
#undef CSA_COMPRESS_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
