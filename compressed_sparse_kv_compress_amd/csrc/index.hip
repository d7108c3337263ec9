// Lightning Indexer scores: I(t, s) = sum_h w[t][h] * max(0, q_I[t][h] . k_I[s])
// for every compressed entry s visible to query t (s < floor(t/m)).
//
// Method: shareware.cn Hybrid Attention article, sections 六-七 (a cheap
// scorer with few heads and a small head dim, per-head ReLU before the head
// sum); trdm.cn attention article, section 4.2 (relu of q_idx against the
// pooled index keys, the key shared by all indexer heads).
//
// Design (gfx950, bf16): in decode the scan over all index keys is the
// dominant HBM stream (256 B per key at d_I = 128) while each key costs
// H_I * d_I MACs, i.e. 64 flop per byte at H_I = 64: above the fp32 VALU
// ridge, so the dot products run on MFMA.  One wavefront owns 32 keys at a
// time: A = the query's H_I x d_I indexer block (held in VGPRs for the whole
// kernel), B = 32 keys x d_I loaded straight from HBM into MFMA operand
// layout (no LDS round trip: every key is used by exactly one wavefront),
// v_mfma_f32_32x32x16_bf16 accumulates 32 heads x 32 keys per block.  In the
// 32x32 output layout a lane holds one key column and 16 head rows, so the
// ReLU and the weighted head sum are in-register FMAs plus one cross-half
// lane exchange; the epilogue writes 32 fp32 scores (128 B) per tile.
// Each wavefront keeps three tiles (24 KiB) of keys in flight.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {
namespace {

constexpr int kWaves = 4;
#ifndef CSA_INDEX_TILES
#define CSA_INDEX_TILES 8
#endif
#ifndef CSA_INDEX_DEPTH
#define CSA_INDEX_DEPTH 3
#endif
constexpr int kTilesPerWave = CSA_INDEX_TILES;  // 32-key tiles streamed by one wavefront
constexpr int kDepth = CSA_INDEX_DEPTH;         // tiles in flight per wavefront
constexpr int kKeysPerWg = kWaves * kTilesPerWave * 32;

template <int MB, int KS, bool HAS_W>
__global__ __launch_bounds__(256) void index_score_mfma(IndexScoreArgs a, int64_t parts) {
  constexpr int HI = 32 * MB;
  constexpr int DI = 16 * KS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t lrow = blockIdx.x / parts;
  const int64_t part = blockIdx.x % parts;
  const int64_t row = a.row0 + lrow;
  const int64_t b = row / a.T;
  const int64_t tpos = a.n_ctx - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  float* srow = a.score + lrow * a.ld;

  const int64_t wave_begin = part * kKeysPerWg + wave * (kTilesPerWave * 32);
  if (wave_begin >= a.L) return;
  const int half = lane >> 5;
  const int col = lane & 31;

  if (wave_begin >= nv) {  // nothing visible in this wavefront's range
    for (int i = 0; i < kTilesPerWave; ++i) {
      const int64_t s = wave_begin + i * 32 + col;
      if (half == 0 && s < a.L) srow[s] = -INFINITY;
    }
    return;
  }

  // Key loads are unconditional (rows past the end are clamped to the last
  // one), so the stream has no control flow and every tile of the prefetch
  // window really is in flight.
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.L * DI + half * 8;
  const int64_t s_last = a.L - 1;
  auto load_tile = [&](int it, bf16x8* frag) {
    int64_t s = wave_begin + it * 32 + col;
    s = s < s_last ? s : s_last;
    const uint16_t* p = kbase + s * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) frag[ks] = *reinterpret_cast<const bf16x8*>(p + ks * 16);
  };
  bf16x8 buf[kDepth][KS];
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) load_tile(i, buf[i]);

  // A operand: query heads (rows) x index dims, resident for the whole kernel.
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + row * HI * DI;
  bf16x8 afrag[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      afrag[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (mb * 32 + col) * DI + ks * 16 + half * 8);

  // Head weights for the 16 head rows this lane holds in each 32x32 block.
  float wr[MB][HAS_W ? 16 : 1];
  if (HAS_W) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < (HAS_W ? 16 : 1); ++r) {
        const int h = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        wr[mb][r] = a.w[row * HI + h];
      }
  }

#pragma unroll
  for (int it = 0; it < kTilesPerWave; ++it) {
    if (it + kDepth - 1 < kTilesPerWave) load_tile(it + kDepth - 1, buf[(it + kDepth - 1) % kDepth]);
    const bf16x8* cur = buf[it % kDepth];
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[mb][ks], cur[ks], acc[mb], 0, 0, 0);
    float part_sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float rl = fmaxf(acc[mb][r], 0.f);
        part_sum = HAS_W ? fmaf(wr[mb][HAS_W ? r : 0], rl, part_sum) : part_sum + rl;
      }
    part_sum += __shfl_xor(part_sum, 32, 64);
    const int64_t s = wave_begin + it * 32 + col;
    const float val = s < nv ? part_sum : -INFINITY;
    if (half == 0 && s < a.L) srow[s] = val;
  }
}

// fp32 storage: VALU dot products in fp32 (small indexer shapes).
__global__ __launch_bounds__(256) void index_score_f32(IndexScoreArgs a, int64_t parts) {
  extern __shared__ float qs[];
  const int64_t lrow = blockIdx.x / parts;
  const int64_t part = blockIdx.x % parts;
  const int64_t row = a.row0 + lrow;
  const int64_t b = row / a.T;
  const int64_t tpos = a.n_ctx - a.T + row % a.T;
  int64_t nv = tpos / a.m;
  if (nv > a.L) nv = a.L;
  const float* q = static_cast<const float*>(a.q) + row * a.HI * a.dI;
  for (int64_t i = threadIdx.x; i < a.HI * a.dI; i += blockDim.x) qs[i] = q[i];
  __syncthreads();
  const int64_t s = part * blockDim.x + threadIdx.x;
  if (s >= a.L) return;
  float* srow = a.score + lrow * a.ld;
  if (s >= nv) {
    srow[s] = -INFINITY;
    return;
  }
  const float* kr = static_cast<const float*>(a.k) + (b * a.L + s) * a.dI;
  float tot = 0.f;
  for (int64_t h = 0; h < a.HI; ++h) {
    float dot = 0.f;
    for (int64_t c = 0; c < a.dI; ++c) dot = fmaf(qs[h * a.dI + c], kr[c], dot);
    const float wh = a.w ? a.w[row * a.HI + h] : 1.0f;
    tot = fmaf(wh, fmaxf(dot, 0.f), tot);
  }
  srow[s] = tot;
}

}  // namespace

hipError_t launch_index_score(const IndexScoreArgs& a, bool bf16, hipStream_t s) {
  if (a.nrows == 0 || a.L == 0) return hipSuccess;
  if (bf16) {
    const int64_t parts = (a.L + kKeysPerWg - 1) / kKeysPerWg;
    const dim3 grid(static_cast<uint32_t>(a.nrows * parts));
    const int mb = static_cast<int>(a.HI / 32), ks = static_cast<int>(a.dI / 16);
    const bool w = a.w != nullptr;
#define CSA_INDEX_LAUNCH(MB_, KS_)                                                                    \
  if (mb == MB_ && ks == KS_) {                                                                       \
    if (w) hipLaunchKernelGGL((index_score_mfma<MB_, KS_, true>), grid, dim3(256), 0, s, a, parts);   \
    else hipLaunchKernelGGL((index_score_mfma<MB_, KS_, false>), grid, dim3(256), 0, s, a, parts);    \
  } else
    CSA_INDEX_LAUNCH(2, 8)
    CSA_INDEX_LAUNCH(1, 8)
    CSA_INDEX_LAUNCH(2, 4)
    CSA_INDEX_LAUNCH(1, 4)
    CSA_INDEX_LAUNCH(4, 8)
    { return hipErrorInvalidValue; }
#undef CSA_INDEX_LAUNCH
  } else {
    const int64_t parts = (a.L + 255) / 256;
    const size_t lds = static_cast<size_t>(a.HI * a.dI) * sizeof(float);
    hipLaunchKernelGGL(index_score_f32, dim3(static_cast<uint32_t>(a.nrows * parts)), dim3(256), lds, s,
                       a, parts);
  }
  return hipGetLastError();
}

bool index_shape_supported(int64_t HI, int64_t dI, bool bf16) {
  if (!bf16) return HI * dI * 4 <= 65536;
  const int64_t mb = HI / 32, ks = dI / 16;
  if (HI % 32 || dI % 16) return false;
  return (ks == 8 && (mb == 1 || mb == 2 || mb == 4)) || (ks == 4 && (mb == 1 || mb == 2));
}

}  // namespace csa
