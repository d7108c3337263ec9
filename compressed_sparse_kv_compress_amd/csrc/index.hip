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
// ridge, so the dot products run on MFMA.  One wavefront owns 16 keys at a
// time: A = the query's H_I x d_I indexer block (held in VGPRs for the whole
// kernel), B = 16 keys x d_I loaded straight from HBM into MFMA operand
// layout (no LDS round trip: every key is used by exactly one wavefront),
// v_mfma_f32_16x16x32_bf16 accumulates 16 heads x 16 keys per block.  In the
// 16x16 output layout a lane holds one key column and 4 head rows per block,
// so the ReLU and the weighted head sum are in-register FMAs plus two lane
// exchanges; the epilogue writes 16 fp32 scores (64 B) per tile.
// Each wavefront keeps three tiles (24 KiB) of keys in flight.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {
namespace {

constexpr int kWaves = 4;
#ifndef CSA_INDEX_TILES
#define CSA_INDEX_TILES 16
#endif
#ifndef CSA_INDEX_DEPTH
#define CSA_INDEX_DEPTH 3
#endif
#ifndef CSA_INDEX_NT
#define CSA_INDEX_NT 1
#endif
constexpr int kTileKeys = 16;                   // keys per MFMA tile (the N dimension)
constexpr int kTilesPerWave = CSA_INDEX_TILES;  // tiles streamed by one wavefront
constexpr int kDepth = CSA_INDEX_DEPTH;         // tiles in flight per wavefront
constexpr int kKeysPerWg = kWaves * kTilesPerWave * kTileKeys;

// MB = H_I / 16 head blocks (the M dimension), KS = d_I / 32 k-steps.
// Only d_I = 128 (KS = 4: one key = 16 granules of 16 B) uses the coalesced
// LDS re-layout below; it is the shape of every CSA configuration.
template <int MB, int KS, bool HAS_W>
__global__ __launch_bounds__(256) void index_score_mfma(IndexScoreArgs a, int64_t parts) {
  constexpr int HI = 16 * MB;
  constexpr int DI = 32 * KS;
  constexpr int GRAN = DI / 8;                 // 16-byte granules per key
  constexpr int TILE_BYTES = kTileKeys * DI * 2;
  constexpr int LOADS = TILE_BYTES / 1024;     // 1 KiB wave-wide loads per tile
  static_assert(GRAN == 16 && LOADS == 4, "coalesced tile layout assumes d_I = 128");
  __shared__ __attribute__((aligned(16))) uint32_t lds[kWaves][2][TILE_BYTES / 4];
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

  const int64_t wave_begin = part * kKeysPerWg + wave * (kTilesPerWave * kTileKeys);
  if (wave_begin >= a.L) return;
  const int g = lane >> 4;    // 16-lane group: k-slots 8g .. 8g+7 of every k-step
  const int c16 = lane & 15;  // key column within the tile

  if (wave_begin >= nv) {  // nothing visible in this wavefront's range
    for (int i = 0; i < kTilesPerWave; ++i) {
      const int64_t s = wave_begin + i * kTileKeys + c16;
      if (g == 0 && s < a.L) srow[s] = -INFINITY;
    }
    return;
  }

  // Coalesced key stream: load i of a tile covers keys 4i .. 4i+3 (1 KiB
  // contiguous); lane l holds granule l%16 of key 4i + l/16.  Loads are
  // unconditional (rows past the end are clamped to the last one), so the
  // stream has no control flow and the whole prefetch window is in flight.
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.L * DI;
  const int64_t s_last = a.L - 1;
  auto load_tile = [&](int it, u32x4* frag) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int64_t s = wave_begin + it * kTileKeys + 4 * i + g;
      s = s < s_last ? s : s_last;
      const u32x4* p = reinterpret_cast<const u32x4*>(kbase + s * DI) + c16;
      frag[i] = CSA_INDEX_NT ? __builtin_nontemporal_load(p) : *p;
    }
  };
  u32x4 buf[kDepth][LOADS];
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) load_tile(i, buf[i]);

  // A operand: query heads (rows) x index dims, resident for the whole kernel.
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + row * HI * DI;
  bf16x8 afrag[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      afrag[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (mb * 16 + c16) * DI + ks * 32 + g * 8);

  // Head weights for the 4 head rows this lane holds in each 16x16 block.
  float wr[MB][HAS_W ? 4 : 1];
  if (HAS_W) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < (HAS_W ? 4 : 1); ++r) wr[mb][r] = a.w[row * HI + mb * 16 + 4 * g + r];
  }

#pragma unroll
  for (int it = 0; it < kTilesPerWave; ++it) {
    if (it + kDepth - 1 < kTilesPerWave) load_tile(it + kDepth - 1, buf[(it + kDepth - 1) % kDepth]);
    // Re-layout through a wave-private LDS tile.  Granule p of key kk sits in
    // slot kk*16 + (p ^ kk): the stores (16 lanes per key) and the MFMA-layout
    // loads (16 keys per granule) both touch 16 distinct bank groups.
    uint32_t* t = lds[wave][it & 1];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int kk = 4 * i + g;
      *reinterpret_cast<u32x4*>(t + 4 * (kk * 16 + (c16 ^ kk))) = buf[it % kDepth][i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bf16x8 cur[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      cur[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t + 4 * (c16 * 16 + ((4 * ks + g) ^ c16))));
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[mb][ks], cur[ks], acc[mb], 0, 0, 0);
    // lane holds S[head mb*16 + 4g + r][key c16]: ReLU, head weights, and the
    // sum over heads (in-lane, then across the four lane groups).
    float part_sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rl = fmaxf(acc[mb][r], 0.f);
        part_sum = HAS_W ? fmaf(wr[mb][HAS_W ? r : 0], rl, part_sum) : part_sum + rl;
      }
    part_sum += __shfl_xor(part_sum, 16, 64);
    part_sum += __shfl_xor(part_sum, 32, 64);
    const int64_t s = wave_begin + it * kTileKeys + c16;
    const float val = s < nv ? part_sum : -INFINITY;
    if (g == 0 && s < a.L) srow[s] = val;
  }
}

// Other d_I (64): MFMA operands straight from global memory (64 B per key
// per load instruction).
template <int MB, int KS, bool HAS_W>
__global__ __launch_bounds__(256) void index_score_mfma_direct(IndexScoreArgs a, int64_t parts) {
  constexpr int HI = 16 * MB;
  constexpr int DI = 32 * KS;
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
  const int64_t wave_begin = part * kKeysPerWg + wave * (kTilesPerWave * kTileKeys);
  if (wave_begin >= a.L) return;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.L * DI + g * 8;
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + row * HI * DI;
  bf16x8 afrag[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      afrag[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (mb * 16 + c16) * DI + ks * 32 + g * 8);
  for (int it = 0; it < kTilesPerWave; ++it) {
    int64_t s = wave_begin + it * kTileKeys + c16;
    const int64_t sc = s < a.L - 1 ? s : a.L - 1;
    bf16x8 cur[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cur[ks] = *reinterpret_cast<const bf16x8*>(kbase + sc * DI + ks * 32);
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[mb][ks], cur[ks], acc[mb], 0, 0, 0);
    float part_sum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rl = fmaxf(acc[mb][r], 0.f);
        part_sum = HAS_W ? fmaf(a.w[row * HI + mb * 16 + 4 * g + r], rl, part_sum) : part_sum + rl;
      }
    part_sum += __shfl_xor(part_sum, 16, 64);
    part_sum += __shfl_xor(part_sum, 32, 64);
    const float val = s < nv ? part_sum : -INFINITY;
    if (g == 0 && s < a.L) srow[s] = val;
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
    const int mb = static_cast<int>(a.HI / 16), ks = static_cast<int>(a.dI / 32);
    const bool w = a.w != nullptr;
#define CSA_INDEX_LAUNCH(K_, MB_, KS_)                                                                \
  if (mb == MB_ && ks == KS_) {                                                                       \
    if (w) hipLaunchKernelGGL((K_<MB_, KS_, true>), grid, dim3(256), 0, s, a, parts);                 \
    else hipLaunchKernelGGL((K_<MB_, KS_, false>), grid, dim3(256), 0, s, a, parts);                  \
  } else
    CSA_INDEX_LAUNCH(index_score_mfma, 4, 4)
    CSA_INDEX_LAUNCH(index_score_mfma, 2, 4)
    CSA_INDEX_LAUNCH(index_score_mfma, 8, 4)
    CSA_INDEX_LAUNCH(index_score_mfma, 1, 4)
    CSA_INDEX_LAUNCH(index_score_mfma_direct, 4, 2)
    CSA_INDEX_LAUNCH(index_score_mfma_direct, 2, 2)
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
  if (HI % 16 || dI % 32) return false;
  const int64_t mb = HI / 16, ks = dI / 32;
  return (ks == 4 && (mb == 1 || mb == 2 || mb == 4 || mb == 8)) || (ks == 2 && (mb == 2 || mb == 4));
}

}  // namespace csa
