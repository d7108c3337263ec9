// Internal launch interface between the C-ABI layer and the gfx950 kernels.
// Arguments are validated by the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// Storage types, numbered as csa_dtype_t: fp32, bf16, and FP8 (OCP E4M3).
enum Dt : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kMXFP4 = 3 };

struct CompressArgs {
  const void* x_a;
  const void* z_a;
  const void* x_b;  // null: single path
  const void* z_b;
  const float* bias;  // null or [span][D]
  void* out;          // [B][out_ld][D], entry j at row j - e0
  int64_t B, n, D, m, p0, n_raw, e0, e1, out_ld;
};
hipError_t launch_compress(const CompressArgs& a, Dt dt, hipStream_t s);

struct IndexScoreArgs {
  const void* q;      // [rows][HI][dI], rows = B*T (b-major)
  const float* w;     // [rows][HI] or null
  const void* k;      // [B][L][dI]
  float* score;       // [rows][ld]
  int64_t ld;
  int64_t row0;       // first (b,t) row handled by this launch
  int64_t nrows;      // rows handled
  int64_t B, T, n_ctx, L, HI, dI, m;
  Dt dt;              // storage of q and k (scores are fp32)
};
hipError_t launch_index_score(const IndexScoreArgs& a, hipStream_t s);

// Per-part top-k candidates: part p of row r keeps ccnt[r][p] <= cap
// (score, index) pairs in index order at [r][p][0 ..]; slots past them hold
// NaN scores.  Optionally (lval != nullptr) a compact list per part: at
// least its lrank largest scores and every score >= the smallest listed one,
// lthr[r][p], in index order, lcnt[r][p] <= lcap of them; lcnt = -1 when
// there is no list (it would be longer, the part has at most cap entries, or
// its selection took the radix path): then the merge reads the full
// candidates.
struct IndexCandidates {
  float* cval;    // [rows][parts][cap]
  int32_t* cidx;  // [rows][parts][cap]
  int32_t* ccnt;  // [rows][parts]
  int64_t cap;
  float* lval = nullptr;    // [rows][parts][lcap]
  int32_t* lidx = nullptr;  // [rows][parts][lcap]
  int32_t* lcnt = nullptr;  // [rows][parts]
  float* lthr = nullptr;    // [rows][parts]
  int64_t lrank = 0, lcap = 0;
};
// Geometry of the streaming indexer (d_I = 128, bf16): key-range parts per
// row (one workgroup each) and keys per wavefront.
void index_plan(int64_t nrows, int64_t L, int64_t* parts, int64_t* per_wave);

struct TopkArgs {
  const float* score;  // row r of this launch at score + r*ld
  int64_t ld;
  int64_t row0;        // global (b,t) row of the first row (for positions)
  int64_t nrows;
  int64_t T, n_ctx, L, m, k;
  int32_t* idx;        // [rows][k] (offset to row0 already)
  float* out_score;    // [rows][k] or null
};
// ws: topk_ws_bytes_per_row(L, k) bytes per row of the launch.
size_t topk_ws_bytes_per_row(int64_t L, int64_t k);
hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t s);
// Merge stage alone over part candidates (fast path: nparts * cap <= 16384,
// nparts <= 256).  fused: the candidates cover every visible entry of rows
// with at most k of them (there is no score matrix to read).
hipError_t launch_topk_merge(const TopkArgs& a, int64_t nparts, const IndexCandidates& c, bool fused, hipStream_t s);
// Compact-list geometry for nparts parts and top-k: the rank (0: no lists)
// and the list capacity.  The merge stages at most kMergeUnion list entries.
constexpr int64_t kMergeUnion = 4096;
inline void compact_list_plan(int64_t nparts, int64_t k, int64_t* lrank, int64_t* lcap) {
  const int64_t r = (2 * k + nparts - 1) / nparts;  // the lists hold at least 2k entries in all
  if (nparts < 4 || 4 * r > k || nparts * 2 * r > kMergeUnion) {
    *lrank = 0;
    *lcap = 0;
    return;
  }
  *lrank = r;
  *lcap = 2 * r;
}

// Indexer scan fused with the part stage of the top-k (no score matrix): the
// scan's workgroups select their parts' candidates from LDS, then the merge
// runs.  Available for bf16 and FP8, d_I = 128, k <= 2048 when the scan's
// parts give the merge's fast path; ws: index_topk_fused_ws_bytes(nrows, L, k).
// Prefill scoring of 16 rows per workgroup (bf16, d_I = 128, H_I <= 64)
// applies to a launch of rows [row0, row0 + nrows) when every sequence has
// T >= 64 queries with T, row0 and nrows multiples of 16.
bool index_multi_rows(int64_t T, int64_t HI, int64_t row0, int64_t nrows);
bool index_topk_fusable(int64_t nrows, int64_t L, int64_t HI, int64_t dI, int64_t k, Dt dt);
size_t index_topk_fused_ws_bytes(int64_t nrows, int64_t L, int64_t k);
hipError_t launch_index_topk_fused(const IndexScoreArgs& a, const TopkArgs& t, void* ws, hipStream_t s);

struct AttnArgs {
  const void* q;        // [B*T][H][d]
  const void* kc;       // [B][L][d]
  const void* vc;
  int64_t L, m;
  const int32_t* idx;   // sparse: [B*T][k]; dense: null
  int64_t k;
  const void* kr;       // [B][R][d], positions n_ctx-R .. n_ctx-1
  const void* vr;
  int64_t R, W;
  const float* sink;    // [H] or null
  float scale;
  int64_t B, T, n_ctx, H, d;
  void* out;            // [B*T][H][d]
  float* lse;           // [B*T][H] or null
  float* ws;            // split partials
  size_t ws_bytes;
};
// Number of row splits the attention launch uses, and its workspace bytes.
// MFMA attention (bf16, or FP8 K/V with bf16 q and out): at most
// kAttnMaxSplits splits per query (the combine kernel gives one lane to each),
// and a CSA split caches at most kAttnMaxIdx row indices, so a sparse row list
// (k + W) is limited to their product.  dt names the K/V storage type.
constexpr int kAttnMaxSplits = 64;
constexpr int kAttnMaxIdx = 2048;
int attn_splits(int64_t B, int64_t T, int64_t H, int64_t d, int64_t max_rows, Dt dt, bool sparse);
size_t attn_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t d, int nsplit);
hipError_t launch_attn(const AttnArgs& a, bool sparse, Dt dt, int nsplit, hipStream_t s);
bool attn_shape_supported(int64_t H, int64_t d, Dt dt);
bool index_shape_supported(int64_t HI, int64_t dI, Dt dt);

}  // namespace csa
