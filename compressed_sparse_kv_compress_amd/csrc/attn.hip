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
// are dense contractions: MFMA v_mfma_f32_16x16x32_bf16, one wavefront per 16
// heads, four wavefronts (64 heads) per workgroup.  Rows are staged 32 at a
// time straight into LDS with direct-to-LDS loads (two stages in flight),
// gathered through the index list for CSA or streamed contiguously for HCA;
// one staged row serves all 64 heads.  Scores are computed transposed
// (S^T = K Q^T), which leaves every lane holding exactly the P values that the
// A operand of O += P V needs, and the V operand comes from the LDS transpose
// load (ds_read_b64_tr_b16), so neither P nor V is shuffled.  The softmax is
// online in log2 units with a lazily re-based running max; the 16 heads x d
// output accumulators live in VGPRs.  Decode queries are split over the row
// list (flash-decoding) and merged by a log-sum-exp combine kernel that also
// applies the sink; prefill-sized launches use one workgroup per (query, 64
// heads) and finish in place.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {
namespace {

constexpr int kHeadsPerWave = 16;
constexpr int kHeadGroups = 4;                            // 16-head groups per workgroup
constexpr int kWaves = 2 * kHeadGroups;                   // each group split over two halves of d
constexpr int kHeadsPerWg = kHeadsPerWave * kHeadGroups;  // 64

struct RowMap {
  int64_t n_cmp;   // compressed slots (sparse: k, dense: visible count)
  int64_t n_win;   // window rows
  int64_t win_lo;  // first raw position of the window
};

// Rows of query t: a sparse call lists k compressed slots; a dense call (or
// a gathered dense call over a paged cache, idx == null) every visible entry.
__device__ __forceinline__ RowMap row_map(const AttnArgs& a, bool sparse, int64_t t) {
  RowMap r;
  if (sparse && a.idx != nullptr) {
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

// Slot of raw position u in sequence b's window buffer of R rows: u % R for
// a ring, else u - (n_b - R) (the buffer holds positions n_b - R .. n_b - 1).
__device__ __forceinline__ int64_t window_slot(const AttnArgs& a, int64_t n_b, int64_t u) {
  return a.lay.ring ? u % a.R : u - (n_b - a.R);
}

// Element offset of virtual row v of query (b, bt) in its source, or -1 if the
// row is empty.  *from_raw tells which source (compressed cache or window).
__device__ __forceinline__ int64_t row_offset(const AttnArgs& a, bool sparse, const RowMap& rm, int64_t n_b,
                                              int64_t b, int64_t bt, int64_t v, bool* from_raw) {
  if (v < rm.n_cmp) {
    *from_raw = false;
    int64_t s = v;
    if (sparse && a.idx != nullptr) {
      s = a.idx[bt * a.k + v];
      if (s < 0 || s >= a.L) return -1;
    }
    return cache_row(a.lay, a.L, b, s) * a.d;
  }
  const int64_t w = v - rm.n_cmp;
  if (w >= rm.n_win) return -1;
  *from_raw = true;
  return (b * a.R + window_slot(a, n_b, rm.win_lo + w)) * a.d;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 hbf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (low half = a), round to nearest even, on the
// hardware converter (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), hbf16x2));
}

// Split workspace: bf16 partial rows [B*T][nsplit][H][d], then fp32 (m, l)
// pairs [B*T][nsplit][H][2].
__device__ __forceinline__ uint16_t* attn_ws_o(const AttnArgs& a) { return reinterpret_cast<uint16_t*>(a.ws); }
__device__ __forceinline__ float* attn_ws_ml(const AttnArgs& a, int nsplit) {
  return reinterpret_cast<float*>(attn_ws_o(a) + static_cast<int64_t>(a.B * a.T) * nsplit * a.H * a.d);
}

// Staging geometry.  Rows move global -> LDS by direct-to-LDS loads
// (global_load_lds: one wave instruction = 64 lanes x ESZ bytes of one row,
// landing contiguously), 32 rows of K and 32 of V per stage, two stage buffers
// (four for FP8 rows, so as many bytes are in flight); each of the 8 waves
// stages 8 rows.  bf16 rows: K rows are read as MFMA A
// operands (16 rows x 16 bytes per 16-lane group): a pitch of 4 banks past a
// multiple of the bank count keeps them apart.  V rows are read by the LDS
// transpose load (4 rows x 32 bytes per 16-lane group): a pitch of 8 banks
// past a multiple does the same for them.  FP8 rows (E4M3, D bytes): K is
// read 8 bytes per lane (16 rows per 16-lane group) and V by the 8-bit
// transpose load (rows 4g..4g+3 and 16+4g..16+4g+3, 16 bytes each, per
// group); one pitch of 6 banks past a multiple separates both.
template <int D, bool F8>
struct Ring {
  static constexpr int RB = F8 ? D : 2 * D;              // bytes per row
  static constexpr int ESZ = RB == 1024 ? 16 : 4;        // bytes per lane per load
  static constexpr int IPR = RB / (64 * ESZ);            // loads per row
  static constexpr int ROWS = 32;                        // rows per stage
  static constexpr int RPW = 2 * ROWS / kWaves;          // rows staged per wave
  static constexpr int PK = F8 ? RB + 24 : RB + 16;      // K row pitch (bytes)
  static constexpr int PV = F8 ? RB + 24 : RB + 32;      // V row pitch (bytes)
  static constexpr int KBYTES = ROWS * PK;
  static constexpr int STAGE = ROWS * (PK + PV);
  static constexpr int NS = F8 ? 4 : 2;                 // stage buffers (equal bytes in flight)
  static constexpr int NI = RPW * IPR;                   // loads per wave per stage
  static constexpr int DH = D / 2;                       // dims per wave
  static constexpr int OP = DH + 4;                      // epilogue LDS row pitch (floats)
  static constexpr int EPI = kWaves * kHeadsPerWave * OP * 4;
  static constexpr int BYTES = NS * STAGE > EPI ? NS * STAGE : EPI;  // the ring also holds the epilogue tile
  static_assert(IPR * 64 * ESZ == RB, "whole rows per load group");
  static_assert((NS - 1) * NI < 64, "vmcnt range");
};
constexpr int kMaxIdx = kAttnMaxIdx;  // cached row indices per split (CSA)

// Source of every masked row (past the split's end, or a -1 / out-of-range
// index): its logit is masked, so its P is 0, and zeros keep 0 * V finite
// (an FP8 row holding a NaN code would not).  One row of the widest layout.
__device__ __attribute__((aligned(16))) uint8_t kZeroRow[1024];

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `ahead` stages of NI loads each are outstanding.
template <int NI, int NS>
__device__ __forceinline__ void wait_stages(int ahead) {
  static_assert(NS == 2 || NS == 4, "stage buffers");
  if (NS == 4 && ahead >= 3) wait_vmcnt<(NS == 4 ? 3 : 0) * NI>();
  else if (NS == 4 && ahead == 2) wait_vmcnt<(NS == 4 ? 2 : 0) * NI>();
  else if (ahead >= 1) wait_vmcnt<NI>();
  else wait_vmcnt<0>();
}

// Direct global -> LDS load of one row piece: lane i's ESZ bytes at g land at
// LDS byte address lds + ESZ * i (lds wave-uniform, through M0).  NT marks the
// load nontemporal: right for decode, where each row is read once per launch
// (random 1 KiB gathers from HBM measured 6.8 TB/s with it, 6.3 without).  A
// prefill launch re-reads every compressed row for many queries, and its
// cache fits the Infinity Cache: there the default policy keeps rows cached
// (7.3 TB/s against 7.1 for a 143 MB working set).  Issued as
// inline asm on purpose: the compiler does not then see an asynchronous LDS
// write, so it adds no "wait for every outstanding load" before each later LDS
// read (which would drain the prefetch ring); completion is instead awaited
// explicitly (vmcnt) and published with a barrier.  The instruction writes no
// registers, and its address registers are read when it issues.
template <int ESZ, bool NT>
__device__ __forceinline__ void dma_row(const char* g, const uint8_t* lds) {
  typedef const uint8_t __attribute__((address_space(3))) * lds_ptr;
  const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  uint32_t saved;  // M0 is restored, so the compiler's own uses of it are unaffected
  if constexpr (ESZ == 16 && NT)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(la)
                 : "memory");
  else if constexpr (ESZ == 16)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(la)
                 : "memory");
  else if constexpr (NT)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(la)
                 : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(la)
                 : "memory");
}

// Stage loader for one wave: RPW consecutive virtual rows c0 .. of one matrix
// (K or V) go straight into LDS (global_load_lds), IPR loads per row.  All
// addressing is wave-uniform (scalar) except the lane's byte offset.  CSA row
// indices come from the split's index cache with one vector LDS read.  An
// empty row (past the split's end, or a -1 / out-of-range index) is read from
// the dummy row and flagged in okrow (K waves only), so its logit is masked.
// Compressed rows: SPARSE gathers through the split's cached list of cache
// rows (-1 = empty slot), else rows are consecutive from cbase.  Window row v
// is raw slot v + win0, wrapped once by wrap (the ring size, or a bound no
// slot reaches).
template <int D, bool F8, bool SPARSE, bool NT>
__device__ __forceinline__ void issue_rows(const char* cbase, const char* rbase, const char* dummy, const int* sidx,
                                           uint8_t* lds, int pitch, int c0, int n_cmp, int r_begin, int r_end,
                                           int win0, int wrap, int lane, int* okrow) {
  using C = Ring<D, F8>;
  int sv = 0;
  if (SPARSE) {
    const int v = c0 + lane;
    sv = (lane < C::RPW && v < n_cmp && v < r_end) ? sidx[v - r_begin] : 0;
  }
#pragma unroll
  for (int j = 0; j < C::RPW; ++j) {
    const int v = c0 + j;
    const bool cmp = v < n_cmp;
    int s = v;
    if (SPARSE) s = cmp ? __builtin_amdgcn_readlane(sv, j) : 0;
    const bool ok = v < r_end && (!SPARSE || !cmp || s >= 0);
    int wr = v + win0;
    wr = wr >= wrap ? wr - wrap : wr;
    const char* row = cmp ? cbase + static_cast<int64_t>(s) * C::RB : rbase + static_cast<int64_t>(wr) * C::RB;
    const char* src = ok ? row : dummy;
#pragma unroll
    for (int p = 0; p < C::IPR; ++p)
      dma_row<C::ESZ, NT>(src + p * 64 * C::ESZ + lane * C::ESZ, lds + j * pitch + p * 64 * C::ESZ);
  }
  if (okrow && lane < C::RPW) {
    const int v = c0 + lane;
    const bool cmp = v < n_cmp;
    okrow[lane] = v < r_end && (!SPARSE || !cmp || sv >= 0);
  }
}

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  typedef s16x4 __attribute__((address_space(3))) lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 8-bit transpose load: for a 16-lane group, lanes 2j and 2j+1 address the
// two 8-byte halves of a 16-byte piece of row j, and lane c receives byte c
// of the eight rows, row j in byte j.
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
  typedef i32x2 __attribute__((address_space(3))) lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

// Eight E4M3 codes (byte i = element i) to bf16: exact, every E4M3 value is a
// bf16 value (3 of bf16's 7 fraction bits, exponents 2^-9 .. 2^8).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 w) {
  const hbf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, false);
  const hbf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, true);
  const hbf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, false);
  const hbf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One workgroup = 64 heads of one query over one split of its row list;
// wave w takes heads 16(w%4) .. +16 and half w/4 of d.  Per 32-row stage a
// wave computes its half of S^T = K Q^T (rows x 16 heads, two 16x16x32 tiles)
// and adds the other half's partial sums from LDS; both halves then hold the
// same scores bit for bit (one addition, commutative) and run the same
// softmax.  Lane (g, c) holds head c at rows 4g..4g+3 and 16+4g..16+4g+3:
// exactly the A operand of O += P V with k = 32 rows, no data movement.  V's B
// operand comes from the LDS transpose load: for 16-lane group g, lanes
// 4j..4j+3 address row r0+j, 16 dims, and lane c receives dim c of those four
// rows.  Two waves per SIMD hide each other's LDS and MFMA latency.
template <int D, bool F8, bool SPARSE, bool NT>
__global__ __launch_bounds__(512, 1) void attn_mfma(AttnArgs a, int nsplit) {
  using C = Ring<D, F8>;
  constexpr int KSQ = C::DH / 32;  // k-steps of the wave's half of Q K^T
  constexpr int NB = C::DH / 16;   // 16-dim output blocks of the wave
  constexpr float kRebase = 8.f;   // re-base the running max only when it grows by > 2^8
  __shared__ __attribute__((aligned(16))) uint8_t ring[C::BYTES];
  __shared__ __attribute__((aligned(16))) f32x4 xs[kWaves][2][64];  // partial scores
  __shared__ int sidx[SPARSE ? kMaxIdx : 1];
  __shared__ __attribute__((aligned(16))) int okf[C::NS + 1][C::ROWS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = wave % kHeadGroups;  // head group
  const int dh = wave / kHeadGroups;  // half of d
  const int g = lane >> 4;            // 16-lane group
  const int c16 = lane & 15;

  const int64_t hgroups = a.H / kHeadsPerWg;
  int64_t id = blockIdx.x;
  const int split = static_cast<int>(id % nsplit);
  id /= nsplit;
  const int64_t hg = id % hgroups;
  const int64_t bt = id / hgroups;
  const int64_t b = bt / a.T;
  const int64_t n_b = seq_len(a.lay, a.n_ctx, a.T, b);
  const int64_t t = n_b - a.T + bt % a.T;
  const RowMap rm = row_map(a, SPARSE, t);
  const int64_t n_rows = rm.n_cmp + rm.n_win;
  const int64_t per = (n_rows + nsplit - 1) / nsplit;  // rows per split (the last stage may be partial)
  const int64_t r_begin = split * per;
  const int64_t r_end = r_begin + per < n_rows ? r_begin + per : n_rows;

  // Waves 0-3 stage K rows 8w .. 8w+7 of each stage; waves 4-7 the V rows.
  const int mat = wave / (kWaves / 2);
  const int row0 = (wave % (kWaves / 2)) * C::RPW;
  // gathered rows are absolute cache rows; consecutive ones start at sequence b's
  const char* cbase = static_cast<const char*>(mat ? a.vc : a.kc) + (SPARSE ? 0 : b * a.L * C::RB);
  const char* rbase = static_cast<const char*>(mat ? a.vr : a.kr) + b * a.R * C::RB;
  const char* dummy = reinterpret_cast<const char*>(kZeroRow);
  static_assert(C::RB <= static_cast<int>(sizeof(kZeroRow)), "zero row covers a row");
  const int pitch = mat ? C::PV : C::PK;
  const int moff = (mat ? C::KBYTES : 0) + row0 * pitch;
  const int n_cmp = static_cast<int>(rm.n_cmp);
  const int rb0 = static_cast<int>(r_begin), re0 = static_cast<int>(r_end);
  // raw slot of virtual row v is v + win0 (wrapped once for a ring)
  const int win0 = static_cast<int>(window_slot(a, n_b, rm.win_lo) - rm.n_cmp);
  const int wrap = a.lay.ring ? static_cast<int>(a.R) : INT32_MAX;
  const int nst = static_cast<int>((r_end - r_begin + C::ROWS - 1) / C::ROWS);

  // Pipeline over NS stage buffers: K of stage c+NS is issued as soon as
  // every wave is done with QK of stage c (barrier B), V of stage c+NS-1 once
  // every wave is done with PV of stage c-1 (barrier A); K therefore keeps NS
  // stages in flight, V NS-1.  Before the loop every buffer is free, so the
  // first NS stages of both K and V are issued at once (a split of few stages
  // then waits for one gather round trip less).  The row flags have NS+1
  // buffers because K(c+NS) sets them while stage c still reads its own.
  auto issue = [&](int st) {
    issue_rows<D, F8, SPARSE, NT>(cbase, rbase, dummy, sidx, ring + (st % C::NS) * C::STAGE + moff, pitch,
                          rb0 + st * C::ROWS + row0, n_cmp, rb0, re0, win0, wrap, lane,
                          mat ? nullptr : okf[st % (C::NS + 1)] + row0);
  };
  auto prime = [&]() {
    for (int st = 0; st < C::NS; ++st)
      if (st < nst) issue(st);
  };

  // HCA rows need nothing but their position, so the first stages are on
  // their way before Q is even requested; CSA rows need the split's indices
  // (cached in LDS once, so that the staging loop issues no loads into
  // registers, whose waits would also drain the ring), requested right after
  // Q so that both arrive in one round trip.
  if (!SPARSE) prime();
  const int h0 = static_cast<int>(hg * kHeadsPerWg + hq * kHeadsPerWave);
  // Q fragments (B operand of K Q^T): head h0 + c16, dims dh*DH + ks*32 + 8g .. +8.
  bf16x8 qf[KSQ];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (bt * a.H + h0 + c16) * D + dh * C::DH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
  }
  if (SPARSE) {  // cache rows of the split's compressed slots (an implicit 0 .. nv-1 list when idx is null)
    const int64_t ce = r_end < rm.n_cmp ? r_end : rm.n_cmp;
    for (int64_t v = r_begin + threadIdx.x; v < ce; v += 64 * kWaves) {
      const int64_t s = a.idx ? a.idx[bt * a.k + v] : v;
      sidx[v - r_begin] = (s >= 0 && s < a.L) ? static_cast<int>(cache_row(a.lay, a.L, b, s)) : -1;
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (SPARSE) prime();

  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // head c16; m_run is the same in all four groups
  const float sl2 = a.scale * kLog2e;

  for (int c = 0; c < nst; ++c) {
    const int buf = c % C::NS;
    // stages after c already issued for this wave's matrix (K at this point,
    // V after its issue below): they may stay in flight
    const int ahead = C::NS - 1 < nst - 1 - c ? C::NS - 1 : nst - 1 - c;
    if (mat == 0) wait_stages<C::NI, C::NS>(ahead);  // this wave's K rows of stage c
    __syncthreads();  // A: K(c) in LDS; every wave is done with PV(c-1)
    if (mat == 1 && c >= 1 && c + C::NS - 1 < nst) issue(c + C::NS - 1);  // V(NS-1) went with the first stages
    const uint8_t* Ks = ring + buf * C::STAGE;
    const uint8_t* Vs = Ks + C::KBYTES;

    // ---- this half's S^T = K Q^T: two 16-row tiles x 16 heads --------------
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
    // lane (g, c16): row c16 (and 16 + c16), dims dh*DH + 32ks + 8g .. +8
    const uint8_t* kp = Ks + c16 * C::PK + (dh * C::DH + g * 8) * (F8 ? 1 : 2);
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) {
      bf16x8 k0, k1;
      if constexpr (F8) {
        k0 = fp8x8_to_bf16(*reinterpret_cast<const i32x2*>(kp + ks * 32));
        k1 = fp8x8_to_bf16(*reinterpret_cast<const i32x2*>(kp + 16 * C::PK + ks * 32));
      } else {
        k0 = *reinterpret_cast<const bf16x8*>(kp + ks * 64);
        k1 = *reinterpret_cast<const bf16x8*>(kp + 16 * C::PK + ks * 64);
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s1, 0, 0, 0);
    }
    xs[wave][0][lane] = s0;
    xs[wave][1][lane] = s1;
    if (mat == 1) wait_stages<C::NI, C::NS>(ahead);  // this wave's V rows of stage c
    __syncthreads();  // B: V(c) in LDS; every wave is done with K(c)
    if (mat == 0 && c + C::NS < nst) issue(c + C::NS);
    s0 += xs[wave ^ kHeadGroups][0][lane];
    s1 += xs[wave ^ kHeadGroups][1][lane];

    // Online softmax (log2 units) for head c16 over its 8 rows here and the
    // other groups' 24, against a lazily re-based running max.
    const i32x4 ok0 = *reinterpret_cast<const i32x4*>(&okf[c % (C::NS + 1)][4 * g]);
    const i32x4 ok1 = *reinterpret_cast<const i32x4*>(&okf[c % (C::NS + 1)][16 + 4 * g]);
    float sv[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = ok0[r] ? s0[r] * sl2 : -INFINITY;
      sv[4 + r] = ok1[r] ? s1[r] * sl2 : -INFINITY;
    }
    float cm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    cm = group_max4(cm);
    const float mnew = fmaxf(m_run, cm);
    if (__any(m_run != -INFINITY && mnew > m_run + kRebase)) {
      // rare: re-base this head's sum and the output rows (heads 4g+r) to the new max
      const float alpha = m_run == -INFINITY ? 1.f : fast_exp2(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][r] *= ar;
      }
      m_run = mnew;
    }
    if (m_run == -INFINITY) m_run = mnew;  // first rows of this head: nothing to re-base
    const float mu = m_run == -INFINITY ? 0.f : m_run;
    float pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = fast_exp2(sv[j] - mu);
      l_run += pr[j];
    }
    bf16x8 pa;
    {
      u32x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = cvt_bf16x2(pr[2 * u], pr[2 * u + 1]);
      pa = __builtin_bit_cast(bf16x8, w);
    }

    // ---- O += P V over the 32 rows: k slot 8g+j <-> row 4g+j (j < 4) or
    // row 16+4g+(j-4) -------------------------------------------------------
    if constexpr (F8) {
      // lanes 2j, 2j+1 of group g address row 4g+j (j < 4) or 16+4g+(j-4)
      const int j = c16 >> 1;
      const uint8_t* v8 = Vs + (j < 4 ? 4 * g + j : 12 + 4 * g + j) * C::PV + (c16 & 1) * 8 + dh * C::DH;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 bv = fp8x8_to_bf16(lds_tr8(v8 + nb * 16));
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bv, oacc[nb], 0, 0, 0);
      }
    } else {
      const uint8_t* v0 = Vs + (4 * g + (c16 >> 2)) * C::PV + (c16 & 3) * 8 + dh * C::DH * 2;
      const uint8_t* v1 = v0 + 16 * C::PV;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4 lo = lds_tr16(v0 + nb * 32);
        const s16x4 hi = lds_tr16(v1 + nb * 32);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bv, oacc[nb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the ring is reused below

  // ---- epilogue: oacc[nb][r] = O[head 4g+r][dim dh*DH + 16nb + c16] --------
  const float l_tot = group_sum4(l_run);
  float* ot = reinterpret_cast<float*>(ring) + wave * kHeadsPerWave * C::OP;  // this wave's 16 x DH tile
  // One workgroup finishes in place (sink, normalisation, lse); a split
  // writes its unnormalised bf16 rows and (m, l) for the combine kernel.
  float sc = 1.f;  // per head c16
  if (nsplit == 1) {
    const float sig = a.sink ? a.sink[h0 + c16] * kLog2e : -INFINITY;
    const float M = fmaxf(m_run, sig);
    float den = 0.f, f = 0.f;
    if (M != -INFINITY) {
      f = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
      den = l_tot * f + (sig == -INFINITY ? 0.f : fast_exp2(sig - M));
    }
    sc = den > 0.f ? f / den : 0.f;
    if (a.lse && dh == 0 && g == 0) a.lse[bt * a.H + h0 + c16] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
  } else if (dh == 0 && g == 0) {
    float* wml = attn_ws_ml(a, nsplit) + ((bt * nsplit + split) * a.H + h0 + c16) * 2;
    wml[0] = m_run;
    wml[1] = l_tot;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float ir = __shfl(sc, 4 * g + r, 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ot[(4 * g + r) * C::OP + nb * 16 + c16] = oacc[nb][r] * ir;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 16 rows x DH bf16, 8 dims (16 bytes) per lane and step
  uint16_t* ob = nsplit == 1 ? static_cast<uint16_t*>(a.out) + (bt * a.H + h0) * D
                             : attn_ws_o(a) + ((bt * nsplit + split) * a.H + h0) * D;
  ob += dh * C::DH;
#pragma unroll
  for (int it = 0; it < kHeadsPerWave * C::DH / (64 * 8); ++it) {
    const int e = it * 64 * 8 + lane * 8;
    const int hl = e / C::DH, dd = e % C::DH;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(ot + hl * C::OP + dd);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(ot + hl * C::OP + dd + 4);
    u32x4 w;
    w[0] = cvt_bf16x2(x0[0], x0[1]);
    w[1] = cvt_bf16x2(x0[2], x0[3]);
    w[2] = cvt_bf16x2(x1[0], x1[1]);
    w[3] = cvt_bf16x2(x1[2], x1[3]);
    *reinterpret_cast<u32x4*>(ob + hl * D + dd) = w;
  }
}

// Merge split partials: O = sum_s 2^{m_s-M} O_s / (sum_s 2^{m_s-M} l_s + 2^{sig-M}).
// One wavefront per (query, head, chunk of 8 * 64/G dims), four per
// workgroup.  Its lanes form G groups of 64/G lanes; a lane holds 8 output
// dims and group g takes splits g, g+G, g+2G, ...  Every lane requests its
// first 16 splits' 16 bytes of bf16 partial row while the (m, l) pairs are
// read (up to four per lane), so one memory round trip covers 16G splits;
// the groups' sums meet by lane exchange at the end.  The launch takes the
// fewest groups that cover every split in one round trip (G = 1: a whole
// 512-dim row per wavefront; G = 8: 64-dim chunks).
template <int G>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int nsplit) {
  constexpr int LPC = 64 / G;  // lanes per chunk
  constexpr int kGroup = 16;   // splits per lane per round trip
  __shared__ float fac[4][kAttnMaxSplits];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t D = a.d;
  const int64_t chunk = D < 8 * LPC ? D : 8 * LPC;
  const int64_t nq = D / chunk;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + w;
  const int64_t bh = gw / nq;  // (bt, h)
  const int64_t d0 = (gw % nq) * chunk;
  const int64_t bt = bh / a.H;
  const int64_t h = bh % a.H;
  const int grp = lane / LPC;
  const int c = lane % LPC;
  const bool has_dims = c * 8 < chunk;
  const uint16_t* src = attn_ws_o(a) + (bt * nsplit * a.H + h) * D + d0 + (has_dims ? c * 8 : 0);
  const int64_t sstride = a.H * D;
  u32x4 v[kGroup];
#pragma unroll
  for (int q = 0; q < kGroup; ++q) {
    const int sp = grp + G * q;
    v[q] = *reinterpret_cast<const u32x4*>(src + (sp < nsplit ? sp : 0) * sstride);
  }
  const float* wml = attn_ws_ml(a, nsplit) + (bt * nsplit * a.H + h) * 2;
  float ms[kAttnMaxSplits / 64], ls[kAttnMaxSplits / 64];
  float mloc = -INFINITY;
#pragma unroll
  for (int r = 0; r < kAttnMaxSplits / 64; ++r) {
    const int sp = lane + 64 * r;
    ms[r] = sp < nsplit ? wml[sp * a.H * 2] : -INFINITY;
    ls[r] = sp < nsplit ? wml[sp * a.H * 2 + 1] : 0.f;
    mloc = fmaxf(mloc, ms[r]);
  }
  const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  const float M = fmaxf(wave_max(mloc), sig);
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < kAttnMaxSplits / 64; ++r) {
    const float f = (M == -INFINITY || ms[r] == -INFINITY) ? 0.f : fast_exp2(ms[r] - M);
    if (lane + 64 * r < nsplit) fac[w][lane + 64 * r] = f;
    lsum = fmaf(ls[r], f, lsum);
  }
  float den = wave_sum(lsum);
  if (M != -INFINITY && sig != -INFINITY) den += fast_exp2(sig - M);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += G * kGroup) {
    if (s0 > 0) {  // later round trips (more than 16 G splits)
#pragma unroll
      for (int q = 0; q < kGroup; ++q) {
        const int sp = s0 + grp + G * q;
        v[q] = *reinterpret_cast<const u32x4*>(src + (sp < nsplit ? sp : 0) * sstride);
      }
    }
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int sp = s0 + grp + G * q;
      const float fs = sp < nsplit ? fac[w][sp] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[2 * u] = fmaf(lo_bf16(v[q][u]), fs, acc[2 * u]);
        acc[2 * u + 1] = fmaf(hi_bf16(v[q][u]), fs, acc[2 * u + 1]);
      }
    }
  }
#pragma unroll
  for (int off = LPC; off < 64; off *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (has_dims && grp == 0) {
    u32x4 o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = cvt_bf16x2(acc[2 * u] * inv, acc[2 * u + 1] * inv);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + bh * D + d0 + c * 8) = o;
  }
  if (a.lse && lane == 0 && d0 == 0) a.lse[bh] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
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
  const int64_t n_b = seq_len(a.lay, a.n_ctx, a.T, b);
  const int64_t t = n_b - a.T + bt % a.T;
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
    const int64_t off = v < n_rows ? row_offset(a, sparse, rm, n_b, b, bt, v, &raw) : -1;
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

int attn_splits(int64_t B, int64_t T, int64_t H, int64_t d, int64_t max_rows, Dt dt, bool sparse) {
  (void)d;
  // fp32 (and head counts the MFMA kernel does not take) run one workgroup per query
  if (dt == kF32 || H < kHeadsPerWg || B * T <= 0) return 1;
  const int64_t base = B * T * (H / kHeadsPerWg);
  const int64_t target = 256;  // workgroups wanted per launch (one per CU)
  int64_t ns = (target + base - 1) / base;
  // A split writes a partial row per head (64 heads x d, bf16: as many bytes
  // as 32 K/V rows) that the combine reads back: long lists keep at least two
  // 32-row stages per split, short ones (the sparse list) at least one.
  const int64_t min_rows = max_rows >= 2048 ? 64 : 32;
  const int64_t cap = (max_rows + min_rows - 1) / min_rows;
  if (ns > cap) ns = cap;
  if (ns > kAttnMaxSplits) ns = kAttnMaxSplits;
  // A split costs its number of 32-row stages (each a gather round trip);
  // for that many stages per split take the fewest splits: fewer partial rows
  // to write and combine, and fewer workgroups re-reading the query.
  if (ns > 1) {
    const int64_t stages = (max_rows + 31) / 32;
    const int64_t per = (stages + ns - 1) / ns;
    ns = (stages + per - 1) / per;
  }
  if (sparse) {  // a split caches at most kMaxIdx row indices
    const int64_t need = (max_rows + kMaxIdx - 1) / kMaxIdx;
    if (ns < need) ns = need;
  }
  if (ns < 1) ns = 1;
  return static_cast<int>(ns);
}

size_t attn_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t d, int nsplit) {
  if (nsplit <= 1) return 0;
  return static_cast<size_t>(B * T) * nsplit * H * (d * sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t launch_attn(const AttnArgs& a, bool sparse, Dt dt, int nsplit, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  if (dt == kF32) {
    hipLaunchKernelGGL(attn_f32, dim3(static_cast<uint32_t>(a.B * a.T * a.H)), dim3(64),
                       a.d * sizeof(float), s, a, sparse ? 1 : 0);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<uint32_t>(a.B * a.T * (a.H / kHeadsPerWg) * nsplit));
  // One query per sequence (decode): every row is read once, nontemporal.
  // Several (prefill): rows are shared between the queries, cached.
  const bool once = a.T == 1;
#define CSA_ATTN_LAUNCH(D_, F8_)                                                                                 \
  if (sparse && once) hipLaunchKernelGGL((attn_mfma<D_, F8_, true, true>), grid, dim3(64 * kWaves), 0, s, a, nsplit);  \
  else if (sparse) hipLaunchKernelGGL((attn_mfma<D_, F8_, true, false>), grid, dim3(64 * kWaves), 0, s, a, nsplit);    \
  else if (once) hipLaunchKernelGGL((attn_mfma<D_, F8_, false, true>), grid, dim3(64 * kWaves), 0, s, a, nsplit);      \
  else hipLaunchKernelGGL((attn_mfma<D_, F8_, false, false>), grid, dim3(64 * kWaves), 0, s, a, nsplit);
  if (dt == kFP8) {
    if (a.d != 512) return hipErrorInvalidValue;
    CSA_ATTN_LAUNCH(512, true)
  } else {
    switch (a.d) {
      case 128: CSA_ATTN_LAUNCH(128, false) break;
      case 256: CSA_ATTN_LAUNCH(256, false) break;
      case 512: CSA_ATTN_LAUNCH(512, false) break;
      default: return hipErrorInvalidValue;
    }
  }
#undef CSA_ATTN_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  // Lane groups G: the fewest with one memory round trip for all splits
  // (16 G >= nsplit), and at least enough that a group's 64/G lanes of 8
  // dims do not exceed d.
  int G = nsplit <= 16 ? 1 : (nsplit <= 32 ? 2 : (nsplit <= 64 ? 4 : 8));
  const int gmin = static_cast<int>(512 / a.d);
  if (G < gmin) G = gmin;
  const int64_t waves = a.B * a.T * a.H * (a.d * G / 512);
  const dim3 cgrid(static_cast<uint32_t>(waves / 4)), blk(256);
  switch (G) {
    case 1: hipLaunchKernelGGL(attn_combine<1>, cgrid, blk, 0, s, a, nsplit); break;
    case 2: hipLaunchKernelGGL(attn_combine<2>, cgrid, blk, 0, s, a, nsplit); break;
    case 4: hipLaunchKernelGGL(attn_combine<4>, cgrid, blk, 0, s, a, nsplit); break;
    default: hipLaunchKernelGGL(attn_combine<8>, cgrid, blk, 0, s, a, nsplit); break;
  }
  return hipGetLastError();
}

bool attn_shape_supported(int64_t H, int64_t d, Dt dt) {
  if (dt == kF32) return d >= 1 && d <= 512;
  if (dt == kFP8) return H % kHeadsPerWg == 0 && d == 512;
  return H % kHeadsPerWg == 0 && (d == 128 || d == 256 || d == 512);
}

}  // namespace csa
