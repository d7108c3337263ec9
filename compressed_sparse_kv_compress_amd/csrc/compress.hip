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

// MXFP4 output (OCP microscaling FP4; the pages run the indexer's q.k in FP4,
// shareware.cn article, the low-precision item of its list of what is
// compressed).  The compressed values stay fp32 until this point; a block of
// 32 channels of one entry is 4 consecutive lanes' 8 values.  The block
// shares the scale 2^E with E = floor(log2 max|v|) - 2 (2 is the exponent of
// E2M1's largest magnitude, 6 = 1.5 * 2^2), clamped below at -127 (E8M0's
// smallest; an all-zero block takes it), and each value becomes the E2M1 code
// nearest to v / 2^E, ties to the even code, magnitudes past 6 saturating;
// the sign bit is v's own.  v / 2^E is exact (a power-of-two scaling that
// stays normal), so every decision is taken on the fp32 value itself.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  // midpoints between neighbouring magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; a
  // tie goes to the even code: > where the lower code is even, >= otherwise
  const uint32_t c = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                     static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                     static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                     static_cast<uint32_t>(a > 5.f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Writes 8 channels c0 .. c0+7 of row `row` of an MXFP4 tensor of `nrows`
// rows of D channels (codes first, then scales).  Every lane of the
// wavefront must call it (the block maximum is a 4-lane exchange); only
// lanes with `store` set write.
__device__ __forceinline__ void mx4_store(void* base, int64_t nrows, int64_t D, int64_t row, int64_t c0,
                                          const float* v, bool store) {
  uint32_t amax = 0;  // |v| bit patterns order as the magnitudes do
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t b = __float_as_uint(v[c]) & 0x7fffffffu;
    amax = b > amax ? b : amax;
  }
  // lanes 4i .. 4i+3 hold one block: max over xor-1 and xor-2 neighbours
  uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(amax), 0xB1, 0xF, 0xF, false));
  amax = o > amax ? o : amax;
  o = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(amax), 0x4E, 0xF, 0xF, false));
  amax = o > amax ? o : amax;
  // floor(log2 amax) is the biased exponent field less 127 for a normal
  // amax; a subnormal or zero amax clamps to the smallest scale anyway
  int e = static_cast<int>(amax >> 23) - 127 - 2;
  e = e < -127 ? -127 : e;
  uint32_t w = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) w |= e2m1_code(ldexpf(v[c], -e)) << (4 * c);
  if (!store) return;
  uint8_t* p = static_cast<uint8_t*>(base);
  *reinterpret_cast<uint32_t*>(p + (row * D + c0) / 2) = w;
  if ((c0 & 31) == 0) p[nrows * D / 2 + (row * D + c0) / 32] = static_cast<uint8_t>(e + 127);
}

// The candidates of entry j form one virtual list: stream-B tokens
// (j-1)*m .. j*m-1 first (two-path, j >= 1), then stream-A tokens
// j*m .. min((j+1)*m, n)-1.  Candidate i maps to its stream, raw row and
// bias row here.
struct Cands {
  int64_t nb, na, b_lo, a_lo, a_bias0;
};

// Where the raw rows of a bulk call live: row u of sequence b at
// (b * n_raw + u - p0) of the streams.
struct BulkRows {
  const CompressArgs& a;
  int64_t row_base;
  __device__ void operator()(bool from_b, int64_t u, const void** x, const void** z, int64_t* off) const {
    *x = from_b ? a.x_b : a.x_a;
    *z = from_b ? a.z_b : a.z_a;
    *off = row_base + (u - a.p0);
  }
};

// Fold candidates [lo, hi) of the virtual list into the running (max,
// denominator, numerator) of VEC channels.  Logits are in log2 units.  rows
// maps (stream, position) to the row holding it; the arithmetic does not
// depend on where the rows are.
template <typename IO, typename Rows>
__device__ __forceinline__ void fold_range(const CompressArgs& a, const Cands& cd, int64_t lo, int64_t hi,
                                           const Rows& rows, int64_t c0, float* mx, float* den, float* acc) {
  constexpr int VEC = IO::VEC;
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
      const void* xs;
      const void* zs;
      int64_t r;
      rows(from_b, u, &xs, &zs, &r);
      IO::load(xs, r * a.D + c0, xv[i]);
      IO::load(zs, r * a.D + c0, lv[i]);
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

// Merge of two partial (max, denominator, numerator) states, the lower
// candidate range first (both lanes of a pair evaluate this same expression,
// so they agree bit for bit).
__device__ __forceinline__ void merge_state(float ml, float dl, float al, float mh, float dh, float ah, float* m,
                                            float* d, float* a) {
  const float M = fmaxf(ml, mh);
  const float fl = ml == -INFINITY ? 0.f : fast_exp2(ml - M);
  const float fh = mh == -INFINITY ? 0.f : fast_exp2(mh - M);
  *m = M;
  *d = fmaf(dl, fl, dh * fh);
  *a = fmaf(al, fl, ah * fh);
}

// Blocks of at least this many tokens fold on 16 lanes per channel group
// when a launch has few entries (a decode-time refresh); bulk launches and
// the per-token append fold every candidate in one thread, in candidate
// order, so an appended entry equals the bulk one bit for bit.
constexpr int kSplitM = 32;
constexpr int kSplits = 16;

// One entry j of one sequence for VEC channels from c0; returns true in the
// lane that holds the result (o).  S = 1: the thread folds every candidate in
// order.  S > 1: the candidates are split over S consecutive lanes whose
// partial states are merged pairwise with lane exchanges.
template <typename IO, int S, typename Rows>
__device__ __forceinline__ bool compress_entry(const CompressArgs& a, const Rows& rows, bool live, int64_t j,
                                               int64_t c0, int slice, float* o) {
  constexpr int VEC = IO::VEC;
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
  if (live && lo < hi) fold_range<IO>(a, cd, lo, hi, rows, c0, mx, den, acc);

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
        merge_state(low ? mx[c] : m2, low ? den[c] : d2, low ? acc[c] : a2, low ? m2 : mx[c], low ? d2 : den[c],
                    low ? a2 : acc[c], &mx[c], &den[c], &acc[c]);
      }
    }
    if (slice != 0) return false;
  }
  if (!live) return false;
#pragma unroll
  for (int c = 0; c < VEC; ++c) o[c] = den[c] > 0.f ? acc[c] / den[c] : 0.f;
  return true;
}

// Bulk: one (entry, 16-byte channel group) per S thread slices.  The kernel
// uses no LDS, so its workgroups can share a CU with an LDS-heavy kernel
// running beside it (the indexer scan holds almost all of a CU's LDS).
// MX: bf16 inputs, MXFP4 entries (S = 1 only: every lane of a block holds a
// result).
template <typename IO, int S, bool MX>
__device__ __forceinline__ void compress_bulk(const CompressArgs& a) {
  static_assert(S >= 1 && S <= 64 && (S & (S - 1)) == 0, "slices: a power of two within a wavefront");
  static_assert(!MX || S == 1, "MXFP4 entries need whole 32-channel blocks in consecutive lanes");
  constexpr int VEC = IO::VEC;
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
  const int64_t c0 = cv * VEC;
  float o[VEC];
  const bool have = compress_entry<IO, S>(a, BulkRows{a, b * a.n_raw}, live, a.e0 + jj, c0, slice, o);
  if constexpr (MX) {
    if (!have) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) o[c] = 0.f;
    }
    mx4_store(a.out, a.B * a.out_ld, a.D, b * a.out_ld + jj, c0, o, have);
  } else if (have) {
    IO::store(a.out, (b * a.out_ld + jj) * a.D + c0, o);
  }
}

template <Dt DT, int S, bool MX = false>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  compress_bulk<Io<DT>, S, MX>(a);
}

// Per-token append: where the rows of sequence b live.  The new token
// (position p) is read from the inputs; earlier positions from the staging
// rings (slot u % n_raw).
struct AppendRows {
  const CompressArgs& a;
  int64_t b, p;
  __device__ void operator()(bool from_b, int64_t u, const void** x, const void** z, int64_t* off) const {
    if (u == p) {  // only stream A reads the new token (stream B reads the previous block)
      *x = a.x_a;
      *z = a.z_a;
      *off = b;
      return;
    }
    *x = from_b ? a.ring_xb : a.ring_xa;
    *z = from_b ? a.ring_zb : a.ring_za;
    *off = b * a.n_raw + u % a.n_raw;
  }
};

// One new token per sequence: slice 0 of each channel group stages the
// token's rows (stream A, and stream B in two-path mode) into ring slot
// p % n_raw; when the token completes its block (p + 1 divisible by m) the
// entry p / m is folded from the rings and the new rows and written to the
// cache.  No candidate of that entry occupies slot p % n_raw (n_raw >= 2m in
// two-path mode, >= m otherwise), so the staging store races with no read.
// MX: the rings and new rows are bf16, the cache MXFP4 (every lane of a block
// reaches the store together: the entry flag is uniform over a sequence).
template <Dt DT, int S, bool MX = false>
__global__ __launch_bounds__(256) void compress_append_kernel(CompressArgs a) {
  static_assert(!MX || (DT == kBF16 && S == 1), "MXFP4 entries come from bf16 rows, one lane per channel group");
  constexpr int VEC = Io<DT>::VEC;
  constexpr int LANES = 256 / S;
  const int slice = threadIdx.x % S;
  const int lane = threadIdx.x / S;
  const int64_t nvec = a.D / VEC;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * LANES + lane;
  const bool in = gid < a.B * nvec;
  const int64_t g = in ? gid : 0;
  const int64_t cv = g % nvec;
  const int64_t b = g / nvec;
  const int64_t c0 = cv * VEC;
  const int64_t p = a.pos[b];
  const bool ok = in && p >= 0;  // a negative position stages nothing
  if (ok && slice == 0) {
    const int64_t src = b * a.D + c0, dst = (b * a.n_raw + p % a.n_raw) * a.D + c0;
    float v[VEC];
    Io<DT>::load(a.x_a, src, v);
    Io<DT>::store(a.ring_xa, dst, v);
    Io<DT>::load(a.z_a, src, v);
    Io<DT>::store(a.ring_za, dst, v);
    if (a.x_b) {
      Io<DT>::load(a.x_b, src, v);
      Io<DT>::store(a.ring_xb, dst, v);
      Io<DT>::load(a.z_b, src, v);
      Io<DT>::store(a.ring_zb, dst, v);
    }
  }
  // uniform over the sequence's slices; entries past the cache are not written
  const int64_t j = ok ? p / a.m : 0;
  const bool emit = ok && (p + 1) % a.m == 0 && j < a.out_ld;
  float o[VEC];
  const bool have = compress_entry<Io<DT>, S>(a, AppendRows{a, b, p}, emit, j, c0, slice, o);
  // the block table is read only for an entry that is written (j < L)
  const int64_t row = !have ? 0 : (a.lay.bt ? cache_row(a.lay, a.out_ld, b, j) : b * a.out_ld + j);
  if constexpr (MX) {
    if (!have) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) o[c] = 0.f;
    }
    const int64_t nrows = a.lay.bt ? a.lay.npages * a.lay.page : a.B * a.out_ld;
    mx4_store(a.out, nrows, a.D, row, c0, o, have);
  } else if (have) {
    Io<DT>::store(a.out, row * a.D + c0, o);
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, Dt dt, hipStream_t s) {
  const int vec = dt == kF32 ? 4 : 8;
  const int64_t total = a.B * (a.e1 - a.e0) * (a.D / vec);
  if (total == 0) return hipSuccess;
  // One thread per channel group folds every candidate in order (bulk:
  // wavefronts read whole rows); long blocks (m >= kSplitM) in a launch of
  // few entries (a decode-time refresh) fold on 16 lanes per channel group.
  // MXFP4 entries (bf16 rows in) always fold in one lane per channel group.
  if (dt == kMXFP4) {
    hipLaunchKernelGGL((compress_kernel<kBF16, 1, true>), dim3(static_cast<uint32_t>((total + 255) / 256)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const bool lanes = a.m >= kSplitM && total < 32768;
  const dim3 grid(static_cast<uint32_t>(lanes ? (total + 15) / 16 : (total + 255) / 256));
#define CSA_COMPRESS_LAUNCH(DT_)                                                             \
  if (lanes) hipLaunchKernelGGL((compress_kernel<DT_, kSplits>), grid, dim3(256), 0, s, a);  \
  else hipLaunchKernelGGL((compress_kernel<DT_, 1>), grid, dim3(256), 0, s, a);
  switch (dt) {
    case kBF16: CSA_COMPRESS_LAUNCH(kBF16) break;
    case kFP8: CSA_COMPRESS_LAUNCH(kFP8) break;
    default: CSA_COMPRESS_LAUNCH(kF32) break;
  }
#undef CSA_COMPRESS_LAUNCH
  return hipGetLastError();
}

hipError_t launch_compress_append(const CompressArgs& a, Dt dt, hipStream_t s) {
  const int vec = dt == kF32 ? 4 : 8;
  const int64_t total = a.B * (a.D / vec);
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((total + 255) / 256));
#define CSA_APPEND_LAUNCH(DT_) hipLaunchKernelGGL((compress_append_kernel<DT_, 1>), grid, dim3(256), 0, s, a);
  switch (dt) {
    case kMXFP4: hipLaunchKernelGGL((compress_append_kernel<kBF16, 1, true>), grid, dim3(256), 0, s, a); break;
    case kBF16: CSA_APPEND_LAUNCH(kBF16) break;
    case kFP8: CSA_APPEND_LAUNCH(kFP8) break;
    default: CSA_APPEND_LAUNCH(kF32) break;
  }
#undef CSA_APPEND_LAUNCH
  return hipGetLastError();
}

// Raw window rows of one new token per sequence: position p goes to ring
// slot p % R.  One thread per 16 bytes of a row.
__global__ __launch_bounds__(256) void window_append_kernel(const uint4* k_new, const uint4* v_new, uint4* kr,
                                                            uint4* vr, const int64_t* pos, int64_t B, int64_t R,
                                                            int64_t row16) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= B * row16) return;
  const int64_t b = gid / row16, c = gid % row16;
  const int64_t p = pos[b];
  if (p < 0) return;
  const int64_t dst = (b * R + p % R) * row16 + c;
  kr[dst] = k_new[gid];
  vr[dst] = v_new[gid];
}

hipError_t launch_window_append(const void* k_new, const void* v_new, void* kr, void* vr, const int64_t* pos,
                                int64_t B, int64_t R, int64_t row_bytes, hipStream_t s) {
  const int64_t row16 = row_bytes / 16, total = B * row16;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(window_append_kernel, dim3(static_cast<uint32_t>((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), static_cast<uint4*>(kr),
                     static_cast<uint4*>(vr), pos, B, R, row16);
  return hipGetLastError();
}

}  // namespace csa
