// Fused alpha-entmax attention for AMD Instinct MI355X (gfx950, CDNA4).
//
// Method (AdaSplash pages, cited by title and section):
//  * "AdaSplash: Adaptive Sparse Flash Attention" (ICML 2025 talk summary),
//    "Accelerated Alpha-Entmax Transformation": tau is the root of
//    f(tau) = sum_j [x_j - tau]_+^beta - 1; its derivatives are shifted powers
//    times constants, so Halley steps are cheap, and a bisection bracket is
//    kept so that a Halley step leaving the bracket is replaced by a midpoint.
//  * Same page, "AdaSplash: Fused GPU Kernel for Attention": one workgroup per
//    query tile, the Q tile stays on chip, K tiles are streamed and the row
//    sums of f and its derivatives are accumulated; a second pass streams K/V
//    and accumulates P V.  S and P never reach HBM.
//  * Same page, "Exploiting Sparsity": all-zero probability tiles are skipped
//    (their K/V loads and their MFMA work) in the output pass and backward.
//  * "AdaSplash-2: The Transformer Revolution We Didn't See Coming", "Sparse
//    Attention Makes Waves": a coarse per-row histogram of scores kept in
//    on-chip memory initialises tau so that one or two refinements suffice.
//
// MI355X design (not the pages' Triton design):
//  * MFMA v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2_f32).
//    Scores are computed transposed, S^T = K Q^T: the 32 MFMA output columns
//    are queries, so every lane owns one query and per-row sums of f, f', f''
//    and histogram updates stay inside the lane; only lanes l and l^32 share
//    a row.  The same register tile, converted to bf16, is the B operand of
//    O^T = V^T P^T, whose A operand is read down the columns of the staged V
//    rows with ds_read_b64_tr_b16 (keys permuted consistently), so P never
//    leaves registers.
//  * t = clamp((alpha-1)/sqrt(d) * acc - tau, 0, 1) is one v_fma_f32 with the
//    clamp modifier: tau >= max(x) - 1 keeps every t <= 1.
//  * The first sweep (k_rowmax16 for bf16: 16x16x32 MFMA, sixteen independent
//    accumulators per wave, K tiles loaded straight into XOR-swizzled LDS)
//    takes only row maxima and each row's maximum over every 64-key tile.
//    Tiles whose maximum cannot exceed a row's lower bracket end can never
//    hold a nonzero probability, so the histogram and Halley sweeps visit
//    candidate tiles only; the tile maxima also raise the lower bracket end.
//  * The histogram holds integer moments (count, sum y, sum y^2 of
//    y = x - lo in 2^-24 fixed point) updated with LDS integer atomics, so it is
//    deterministic and, for alpha in {1.5, 2}, gives f exactly at bin edges.
//  * The sparse kernels stage d = 128 bf16 tiles with buffer_load ... lds
//    (no staging registers) and keep LDS reads several MFMA steps ahead.
//  * For bf16 the tau kernel ends with the P V pass over its final mask
//    (kept as bits in LDS), so Q, tau and the mask need no second start-up.
//  * Causal query tiles of the row-max sweep are paired (t, n - 1 - t) per
//    workgroup when that evens out the rounds of resident workgroups.
//  * The dQ kernel leaves the block mask transposed in the workspace, so the
//    dK/dV kernel reads each key tile's active query rows contiguously.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <float.h>

#include <climits>
#include <type_traits>

#include "entmax_attn.h"

namespace {

constexpr int kWave = 64;
constexpr int kBQ = 32;               // queries per wave = mask row granularity
constexpr int kWaves = 4;
constexpr int kBQW = kBQ * kWaves;    // queries per workgroup (forward, dQ)
constexpr int kBK = 64;               // keys per tile = mask column granularity
constexpr int kThreads = kWave * kWaves;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

enum AlphaKind { AK15 = 0, AK20 = 1, AK125 = 2, AKGEN = 3 };

struct Params {
  int N, n_kt, n_q32, causal;
  int Np;                 // N rounded up to 64 (row length of transposed copies)
  int BH;                 // batch * heads
  float alpha, beta, scale, inv_sqrt_d;
  int mode, max_iters, flags;
  float tol;
  int out_bf16;
  int pair_qt;            // row-max sweep: one workgroup per pair of causal query tiles
};

// ----------------------------------------------------------- fragments ---
// A fragment is the 8 consecutive contraction elements one lane feeds to one
// 32x32 MFMA step of 16 (bf16: one instruction; fp32: eight 32x32x2 steps).
template <typename E> struct Frag;
template <> struct Frag<__bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 a, b; };

__device__ __forceinline__ void frag_zero(Frag<__bf16>& f) {
  f.v = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
}
__device__ __forceinline__ void frag_zero(Frag<float>& f) {
  f.a = f32x4{0, 0, 0, 0};
  f.b = f32x4{0, 0, 0, 0};
}
__device__ __forceinline__ void ld8(Frag<__bf16>& f, const __bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void ld8(Frag<float>& f, const float* p) {
  f.a = *reinterpret_cast<const f32x4*>(p);
  f.b = *reinterpret_cast<const f32x4*>(p + 4);
}
// two runs of 4 consecutive elements (transposed tiles, permuted key order)
__device__ __forceinline__ void ld4x2(Frag<__bf16>& f, const __bf16* p0, const __bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void ld4x2(Frag<float>& f, const float* p0, const float* p1) {
  f.a = *reinterpret_cast<const f32x4*>(p0);
  f.b = *reinterpret_cast<const f32x4*>(p1);
}
// LDS row stride (bytes) of a tile of D-element rows.  bf16 rows are padded by
// 48 bytes: consecutive rows then start 48 bytes apart modulo the 256-byte bank
// period, which keeps both access patterns used on these tiles conflict free
// (16 lanes reading 16 rows with ds_read_b128, and 32 lanes reading 4 rows x
// 64 bytes with ds_read_b64_tr_b16).  fp32 rows are padded by 16 bytes.
template <typename E, int D>
constexpr int row_stride() { return D * (int)sizeof(E) + (sizeof(E) == 2 ? 48 : 16); }

// Operand fragment whose 8 contraction elements run down one column of a
// row-major bf16 LDS tile: rows r0 + {0,1,2,3} and r0 + 8 + {0,1,2,3} (the
// permuted key order of the score accumulators), column col0 + (lane & 31).
// ds_read_b64_tr_b16 gives lane i of each 16-lane group element i % 4 of the
// 8-byte chunks addressed by lanes 4j + i / 4 of that group (j = 0..3), so
// lane r of a group addresses row r0 + r / 4, column col0 + 16 * half + 4 * (r % 4).
__device__ __forceinline__ void ld_col8(Frag<__bf16>& f, const char* tile, int rs, int r0, int col0,
                                        int lane) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int g = lane & 15;
  const char* p = tile + (r0 + (g >> 2)) * rs + (col0 + 16 * ((lane >> 4) & 1) + 4 * (g & 3)) * 2;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 8 * rs));
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ float frag_get(const Frag<__bf16>& f, int j) { return (float)f.v[j]; }
__device__ __forceinline__ float frag_get(const Frag<float>& f, int j) { return j < 4 ? f.a[j] : f.b[j - 4]; }
// accumulator registers r[0..7] -> operand fragment
__device__ __forceinline__ void from_acc(Frag<__bf16>& f, const f32x16& acc, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (__bf16)acc[base + j];
}
__device__ __forceinline__ void from_acc(Frag<float>& f, const f32x16& acc, int base) {
  f.a = f32x4{acc[base + 0], acc[base + 1], acc[base + 2], acc[base + 3]};
  f.b = f32x4{acc[base + 4], acc[base + 5], acc[base + 6], acc[base + 7]};
}
// hi/lo bf16 pair: x = hi + lo to about 2^-17 relative (hi = bf16(x), lo = bf16(x - hi);
// x - hi is exact in fp32).  For fp32 fragments lo is unused.
__device__ __forceinline__ void split_acc(Frag<__bf16>& hi, Frag<__bf16>& lo, const f32x16& acc, int base) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    __bf16 hv = (__bf16)acc[base + j];
    hi.v[j] = hv;
    lo.v[j] = (__bf16)(acc[base + j] - (float)hv);
  }
}
__device__ __forceinline__ void split_acc(Frag<float>& hi, Frag<float>&, const f32x16& acc, int base) {
  from_acc(hi, acc, base);
}
template <typename E> constexpr bool kNeedsLo = sizeof(E) == 2;

__device__ __forceinline__ void mma(f32x16& c, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[0], b.a[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[1], b.a[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[2], b.a[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[3], b.a[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[0], b.b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[1], b.b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[2], b.b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[3], b.b[3], c, 0, 0, 0);
}

// Row (M index) held by register i of a 32x32 accumulator in lane-half h;
// the column (N index) is lane & 31.
__device__ __forceinline__ int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ float clamp01(float v) { return __builtin_amdgcn_fmed3f(v, 0.0f, 1.0f); }

// max(x[l], x[l ^ 32]) on every lane, by one v_permlane32_swap
__device__ __forceinline__ float half_swap_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// OR over each 32-lane half of the wave: returns the half-0 result in the low
// and the half-1 result in the high 32 bits (wave-uniform).
__device__ __forceinline__ unsigned long long half_or_dpp(uint32_t v) {
  v |= dpp_u<0xB1>(v);
  v |= dpp_u<0x4E>(v);
  v |= dpp_u<0x141>(v);
  v |= dpp_u<0x140>(v);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0) | (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32) | (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return (unsigned long long)a | ((unsigned long long)b << 32);
}

// ------------------------------------------------------ entmax powers ---
// t in [0, 1].  p = t^beta, u = t^(beta-1) (0 off the support), and the
// sweep sums F0 += t^beta, F1 += t^(beta-1), F2 += t^(beta-2), cnt += [t>0].
template <int AK> struct Ent;
template <> struct Ent<AK15> {   // beta = 2
  __device__ static void sweep(float t, float, float& F0, float& F1, float& F2, float& cnt) {
    F0 = fmaf(t, t, F0);
    F1 += t;
    F2 += ceilf(t);
    (void)cnt;
  }
  __device__ static float count(float, float, float F2, float) { return F2; }
  __device__ static void pu(float t, float, float& p, float& u) { p = t * t; u = t; }
};
template <> struct Ent<AK20> {   // beta = 1 (sparsemax)
  __device__ static void sweep(float t, float, float& F0, float& F1, float&, float&) {
    F0 += t;
    F1 += ceilf(t);
  }
  __device__ static float count(float, float F1, float, float) { return F1; }
  __device__ static void pu(float t, float, float& p, float& u) { p = t; u = ceilf(t); }
};
template <> struct Ent<AK125> {  // beta = 4
  __device__ static void sweep(float t, float, float& F0, float& F1, float& F2, float& cnt) {
    float t2 = t * t;
    F0 = fmaf(t2, t2, F0);
    F1 = fmaf(t2, t, F1);
    F2 += t2;
    cnt += ceilf(t);
  }
  __device__ static float count(float, float, float, float cnt) { return cnt; }
  __device__ static void pu(float t, float, float& p, float& u) {
    float t2 = t * t;
    p = t2 * t2;
    u = t2 * t;
  }
};
template <> struct Ent<AKGEN> {  // any 1 < alpha < 2
  __device__ static void sweep(float t, float beta, float& F0, float& F1, float& F2, float& cnt) {
    float l = log2f(t);
    bool pos = t > 0.0f;
    F0 += exp2f(beta * l);
    F1 += pos ? exp2f((beta - 1.0f) * l) : 0.0f;
    F2 += pos ? exp2f((beta - 2.0f) * l) : 0.0f;
    cnt += ceilf(t);
  }
  __device__ static float count(float, float, float, float cnt) { return cnt; }
  __device__ static void pu(float t, float beta, float& p, float& u) {
    float l = log2f(t);
    p = exp2f(beta * l);
    u = t > 0.0f ? exp2f((beta - 1.0f) * l) : 0.0f;
  }
};

// ------------------------------------------------------- tile staging ---
// S^T for one wave: 64 keys (LDS rows, stride ks) x the wave's 32 queries
// (B fragments in registers).  acc[kb] holds keys 32kb.. as rows.
template <typename E, int D>
__device__ __forceinline__ void scores_T(f32x16 (&acc)[2], const char* klds, int ks,
                                         const Frag<E> (&qf)[D / 16], int lane) {
  const int c32 = lane & 31, h = lane >> 5;
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  // K fragments run three MFMA steps ahead of their use, so an LDS read
  // never stalls the MFMA that consumes it
  constexpr int kSteps = D / 16 * 2, kAhead = 3;
  auto addr = [&](int st) {
    return reinterpret_cast<const E*>(klds + (32 * (st & 1) + c32) * ks) + 16 * (st >> 1) + 8 * h;
  };
  Frag<E> a[kAhead + 1];
#pragma unroll
  for (int st = 0; st < kAhead; ++st) ld8(a[st], addr(st));
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    if (st + kAhead < kSteps) ld8(a[(st + kAhead) % (kAhead + 1)], addr(st + kAhead));
    mma(acc[st & 1], a[st % (kAhead + 1)], qf[st >> 1]);
  }
}

// Visibility limit of this lane's query in an S^T tile whose rows are keys
// key0..key0+63: rows r <= limit are visible (limit < 0: none).  Folding the
// lane-half offset 4h of acc_row() in leaves one compare per element.
__device__ __forceinline__ int row_limit(int key0, int iq, int N, int causal, int h) {
  const int last = iq >= N ? -1 : (causal ? min(iq, N - 1) : N - 1) - key0;
  return last - 4 * h;
}
__device__ __forceinline__ void mask_rows_above(f32x16 (&acc)[2], int lim) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) acc[kb][i] = -INFINITY;
}
// One 32-key half kb of two S^T-shaped tiles at once: sa from the K rows at kl
// with the query fragments qf, pa from the rows at vl with the fragments of.
// The two accumulators are independent MFMA chains, interleaved step by step.
template <typename E, int D>
__device__ __forceinline__ void scores_T_half2(f32x16& sa, f32x16& pa, const char* kl, const char* vl, int ks,
                                               int kb, const Frag<E> (&qf)[D / 16],
                                               const Frag<E> (&of)[D / 16], int lane) {
  const int c32 = lane & 31, h = lane >> 5;
  sa = f32x16{};
  pa = f32x16{};
  const int roff = (32 * kb + c32) * ks;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    Frag<E> a, b;
    ld8(a, reinterpret_cast<const E*>(kl + roff) + 16 * st + 8 * h);
    ld8(b, reinterpret_cast<const E*>(vl + roff) + 16 * st + 8 * h);
    mma(sa, a, qf[st]);
    mma(pa, b, of[st]);
  }
}
// rows (keys) of half kb past the visibility limit of mask_rows_above
__device__ __forceinline__ void mask_half_rows_above(f32x16& acc, int kb, int lim) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) acc[i] = -INFINITY;
}
// Tile of S^T (keys x this wave's 32 queries), masked only when `masked`.
template <typename E, int D, bool M>
__device__ __forceinline__ void tile_scores(f32x16 (&acc)[2], const char* kl, int ks,
                                            const Frag<E> (&qf)[D / 16], int lane, int lim,
                                            std::integral_constant<bool, M>) {
  scores_T<E, D>(acc, kl, ks, qf, lane);
  if constexpr (M) mask_rows_above(acc, lim);
}

template <typename E, int D>
__device__ __forceinline__ void load_qfrags(Frag<E> (&qf)[D / 16], const E* rowp, bool valid, int h) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (valid)
      ld8(qf[c], rowp + 16 * c + 8 * h);
    else
      frag_zero(qf[c]);
  }
}

// --------------------------------------------------- work distribution ---
// Workgroups are dealt round robin to the 8 XCDs (block b runs on XCD b % 8).
// When B*H is a multiple of 8 each XCD gets its own heads, so one XCD's L2
// serves the K/V of few heads; inside an XCD (or globally otherwise) tiles of
// different heads are interleaved by rank.  With heavy_first, rank 0 is the
// tile with the most work (the last query tile when causal).
__device__ __forceinline__ void map_tile(int n_tiles, int BH, bool heavy_first, int& bh, int& tile) {
  const int b = blockIdx.x;
  int rank;
  if ((BH & 7) == 0) {
    const int hx = BH >> 3, j = b >> 3;
    bh = (b & 7) * hx + j % hx;
    rank = j / hx;
  } else {
    bh = b % BH;
    rank = b / BH;
  }
  tile = heavy_first ? n_tiles - 1 - rank : rank;
}

// ---------------------------------------------------- prefetch staging ---
// A tile of ROWS rows x D elements staged global -> registers -> LDS, so the
// global loads of the next tile overlap the MFMA work on the current one.
template <typename E, int D, int ROWS, int NT = kThreads>
struct RowStage {
  static constexpr int CH = D * (int)sizeof(E) / 16;
  static constexpr int PER = (ROWS * CH + NT - 1) / NT;
  f32x4 r[PER];
  __device__ __forceinline__ void load(const E* g, int row0, int N) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c / CH, cc = c - rr * CH;
      const int gr = row0 + rr;
      r[i] = f32x4{0, 0, 0, 0};
      if (c < ROWS * CH && gr < N)
        r[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(g + (size_t)gr * D) + cc * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, int lstride) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c / CH, cc = c - rr * CH;
      if (c < ROWS * CH) *reinterpret_cast<f32x4*>(lds + rr * lstride + cc * 16) = r[i];
    }
  }
};
// Direct global -> LDS staging of a 64-row bf16 tile (buffer_load_dwordx4
// ... lds: lane l of one instruction lands at LDS base + 16 l, no registers
// involved).  Rows are stored unpadded; the 16-byte chunk c of row r sits in
// slot c ^ (r mod chunks-per-row), so the 16 lanes of one ds_read_b128 phase
// that read the same chunk of 16 consecutive rows hit 16 different bank
// groups.  The buffer descriptor spans one head's N rows: rows past N read as
// zeros (the hardware range check), and every reader masks them.
template <int D>
struct DirectTile {
  static constexpr int RB = D * 2;                 // row bytes
  static constexpr int CPR = RB / 16;              // chunks per row
  static constexpr int BYTES = kBK * RB;
  static constexpr int NI = BYTES / 1024 / kWaves; // instructions per wave
  __amdgpu_buffer_rsrc_t rsrc;
  int voff[NI];                                    // this lane's byte offsets in a tile
  __device__ __forceinline__ DirectTile(const __bf16* head, int N, int w, int lane) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(head), (short)0, N * RB, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int p = (w * NI + i) * 1024 + 16 * lane;
      const int r = p / RB, slot = (p % RB) / 16;
      voff[i] = r * RB + ((slot ^ (r & (CPR - 1))) << 4);
    }
  }
  // load key/value rows row0 .. row0+63 into `tile`
  __device__ __forceinline__ void issue(char* tile, int row0, int w) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc,
          reinterpret_cast<__attribute__((address_space(3))) void*>(
              reinterpret_cast<uintptr_t>(tile + (w * NI + i) * 1024)),
          16, voff[i], row0 * RB, 0, 0);
  }
  // address of chunk c (8 elements) of row r
  __device__ __forceinline__ static const __bf16* at(const char* tile, int r, int c) {
    return reinterpret_cast<const __bf16*>(tile + r * RB + ((c ^ (r & (CPR - 1))) << 4));
  }
};
// Wait until at most n vector memory operations of this wave are in flight
// (expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ROWS-row tiles of one head's [N][D] matrix staged into LDS rows of
// row_stride<E, D>() bytes.  fetch(dst, row0) starts the copy of rows
// row0 .. row0+ROWS-1, commit(dst) finishes it; the tile is complete for the
// whole workgroup after the next __syncthreads.  Rows past N read as zeros.
//  - bf16, d = 128: buffer_load_dword ... lds, one instruction per row (64
//    lanes x 4 B) straight into the padded LDS row; no registers hold the
//    tile and commit is empty.  The buffer descriptor spans the head's N
//    rows, so its range check supplies the zeros.
//  - otherwise through registers (RowStage; a d = 64 bf16 tile needs only 8
//    of them per thread), commit writes them to LDS.
template <typename E, int D, int ROWS>
struct RowTiles {
  RowStage<E, D, ROWS> st;
  const E* g;
  int N;
  __device__ __forceinline__ RowTiles(const E* head, int n, int, int) : g(head), N(n) {}
  __device__ __forceinline__ void fetch(char*, int row0) { st.load(g, row0, N); }
  __device__ __forceinline__ void commit(char* dst) const { st.store(dst, row_stride<E, D>()); }
};
template <int ROWS>
struct RowTiles<__bf16, 128, ROWS> {
  static constexpr int D = 128;
  static constexpr int RB = D * 2;                   // bytes of one row in memory
  static constexpr int RS = row_stride<__bf16, D>(); // bytes of one row in LDS
  static constexpr int RPW = ROWS / kWaves;          // rows issued by each wave
  __amdgpu_buffer_rsrc_t rsrc;
  int w, lane;
  __device__ __forceinline__ RowTiles(const __bf16* head, int n, int w_, int lane_)
      : w(__builtin_amdgcn_readfirstlane(w_)), lane(lane_) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(head), (short)0, n * RB, 0x00020000);
  }
  // row0 and dst must be the same for the whole wave (they come from LDS
  // lists, so the compiler is told so: the tile offset goes in an SGPR)
  __device__ __forceinline__ void fetch(char* dst, int row0) {
    const int r0 = __builtin_amdgcn_readfirstlane(row0);
    const uint32_t d0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(dst));
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = w * RPW + r;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(d0 + row * RS), 4, lane * 4,
          (r0 + row) * RB, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(char*) const {}
};

// Columns col0..col0+W of a transposed [D][Np] matrix (all in range).
template <typename E, int D, int W, int NT = kThreads>
struct ColStage {
  static constexpr int CH = W * (int)sizeof(E) / 16;
  static constexpr int PER = (D * CH + NT - 1) / NT;
  f32x4 r[PER];
  __device__ __forceinline__ void load(const E* gt, int Np, int col0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c / CH, cc = c - rr * CH;
      r[i] = f32x4{0, 0, 0, 0};
      if (c < D * CH)
        r[i] = *reinterpret_cast<const f32x4*>(
            reinterpret_cast<const char*>(gt + (size_t)rr * Np + col0) + cc * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, int lstride) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const int rr = c / CH, cc = c - rr * CH;
      if (c < D * CH) *reinterpret_cast<f32x4*>(lds + rr * lstride + cc * 16) = r[i];
    }
  }
};

// Compacts tiles base..base+len-1 whose wave bits (pred(w, t) for the four
// waves) are not all zero into list[] / wbits[]; returns the count.  Every
// thread of the workgroup must call it.  `flags` holds len bytes of scratch.
template <typename Pred>
__device__ __forceinline__ int build_list(int base, int len, Pred pred, short* list, uint8_t* wbits,
                                          uint8_t* flags, int* counter) {
  for (int i = threadIdx.x; i < len; i += kThreads) {
    uint8_t b = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
      if (pred(ww, base + i)) b |= (uint8_t)(1u << ww);
    flags[i] = b;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int count = 0;
    for (int b0 = 0; b0 < len; b0 += kWave) {
      const int i = b0 + lane;
      const uint8_t b = i < len ? flags[i] : 0;
      const unsigned long long bal = __ballot(b != 0);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (b) {
        list[count + before] = (short)i;
        wbits[count + before] = b;
      }
      count += __popcll(bal);
    }
    if (lane == 0) *counter = count;
  }
  __syncthreads();
  return *counter;
}

// Tile maxima are kept as IEEE half bits rounded toward +infinity: the stored
// value bounds the true maximum from above and the half just below it bounds
// it from below (strictly), which is all the pruning and the lower bracket
// end need, at half the bytes of fp32.
// Row length of the tile maxima: whole 64-byte segments (32 tiles), written
// by one lane at once so that no partial segment reaches memory.
__host__ __device__ constexpr int tilemax_row(int n_kt) { return (n_kt + 31) & ~31; }

__device__ __forceinline__ uint16_t half_bits_up(float x) {
  const _Float16 hx = (_Float16)x;
  uint16_t b = __builtin_bit_cast(uint16_t, hx);
  if ((float)hx < x) b = (b & 0x8000u) ? (uint16_t)(b - 1u) : (uint16_t)(b + 1u);
  return b;
}
__device__ __forceinline__ float half_up_value(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// the half just below the stored one (-inf stays -inf)
__device__ __forceinline__ float half_down_value(uint16_t b) {
  uint16_t d;
  if (b == 0xFC00u) d = b;
  else if (b == 0x0000u || b == 0x8000u) d = 0x8001u;
  else d = (b & 0x8000u) ? (uint16_t)(b + 1u) : (uint16_t)(b - 1u);
  return (float)__builtin_bit_cast(_Float16, d);
}

// Each lane collects one row's tile maxima as half bits: the last 8 in a
// 16-byte shift register (oldest lowest), groups of 8 in a SEG-deep queue, and
// stores 8 SEG tiles (16 SEG bytes) at once at the row's position in
// tilemax[bh][row][kt].  Nothing is stored for rows past N (row_ptr null).
template <int SEG>
struct TileMaxQueue {
  static constexpr uint32_t kNegInf2 = 0xFC00FC00u;   // two half -inf
  u32x4 tbuf;
  u32x4 gq[SEG];
  uint16_t* row_ptr;
  __device__ __forceinline__ explicit TileMaxQueue(uint16_t* p) : row_ptr(p) {
    tbuf = u32x4{kNegInf2, kNegInf2, kNegInf2, kNegInf2};
#pragma unroll
    for (int i = 0; i < SEG; ++i) gq[i] = tbuf;
  }
  __device__ __forceinline__ void push(uint32_t hb) {
    tbuf[0] = __builtin_amdgcn_alignbit(tbuf[1], tbuf[0], 16);
    tbuf[1] = __builtin_amdgcn_alignbit(tbuf[2], tbuf[1], 16);
    tbuf[2] = __builtin_amdgcn_alignbit(tbuf[3], tbuf[2], 16);
    tbuf[3] = __builtin_amdgcn_alignbit(hb, tbuf[3], 16);
  }
  __device__ __forceinline__ void push_group() {
#pragma unroll
    for (int i = 0; i + 1 < SEG; ++i) gq[i] = gq[i + 1];
    gq[SEG - 1] = tbuf;
  }
  __device__ __forceinline__ void flush(int kt0) {
    if (row_ptr) {
      u32x4* dst = reinterpret_cast<u32x4*>(row_ptr + kt0);
#pragma unroll
      for (int i = 0; i < SEG; ++i) dst[i] = gq[i];
    }
  }
  // after tile kt's value was pushed; returns true when it stored a segment
  __device__ __forceinline__ bool tile_done(int kt) {
    if ((kt & 7) != 7) return false;
    push_group();
    if (((kt >> 3) % SEG) != SEG - 1) return false;
    flush(kt + 1 - 8 * SEG);
    return true;
  }
  // the last, partial segment after n_done tiles (the rest of it reads -inf)
  __device__ __forceinline__ void finish(int n_done) {
    if (n_done % (8 * SEG) == 0) return;
    if (n_done & 7) {
      for (int r = n_done & 7; r < 8; ++r) push(0xFC00u);
      push_group();
    }
    const int filled = ((n_done + 7) >> 3) % SEG;   // groups queued in the segment
    if (filled) {
      tbuf = u32x4{kNegInf2, kNegInf2, kNegInf2, kNegInf2};
      for (int g = filled; g < SEG; ++g) push_group();
    }
    flush(n_done / (8 * SEG) * (8 * SEG));
  }
};

// ---------------------------------------------------------- k_rowmax ---
// The one full score sweep: per-row maxima of x = (alpha-1) q.k / sqrt(d)
// and, for every row and 64-key tile, the row's maximum x over the tile
// (tilemax[bh][row][kt], rows padded to a multiple of 32 tiles, as half bits
// rounded up; it bounds tau from below and prunes key tiles that can never
// hold a nonzero probability).  Each wave
// owns 64 queries (two B-operand blocks share every K fragment read from
// LDS); the workgroup (256 queries) streams K tiles double-buffered through
// registers.  This 32x32 form serves fp32 inputs; bf16 runs k_rowmax16.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_rowmax(const E* __restrict__ Q, const E* __restrict__ K,
                                                     Params P, float* __restrict__ rowmax,
                                                     uint16_t* __restrict__ tilemax) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int KS = row_stride<E, D>();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = P.N;
  const int n_qt = (N + 255) / 256;
  int bh, qtile;
  map_tile(n_qt, P.BH, P.causal, bh, qtile);
  const int q0 = qtile * 256;
  const int wq0 = q0 + 64 * w;
  const E* Qh = Q + (size_t)bh * N * D;
  const E* Kh = K + (size_t)bh * N * D;

  Frag<E> qf[2][D / 16];
  int iq[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    iq[qb] = wq0 + 32 * qb + c32;
    load_qfrags<E, D>(qf[qb], Qh + (size_t)iq[qb] * D, iq[qb] < N, h);
  }
  const int kt_end = P.causal ? (min(N - 1, q0 + 255) / kBK + 1) : P.n_kt;
  const int kt_end_w = wq0 >= N ? 0 : (P.causal ? (min(N - 1, wq0 + 63) / kBK + 1) : P.n_kt);
  // Tiles below kt_full are fully visible to every query of the workgroup and
  // lie inside [0, N): they need no masking.  Only the diagonal / tail tiles do.
  const int kt_full = min(P.causal ? q0 / kBK : P.n_kt, N / kBK);

  float m[2] = {-INFINITY, -INFINITY};
  RowStage<E, D, kBK> st;
  if (kt_end > 0) {
    st.load(Kh, 0, N);
    st.store(smem, KS);
  }
  __syncthreads();

  const int ktp = tilemax_row(P.n_kt);
  // d = 128 stores 64-byte segments; d = 64 keeps 16-byte stores, which spares
  // the registers of a third wave per SIMD
  constexpr int kSeg = D == 64 ? 1 : 4;
  const int my_row = h ? iq[1] : iq[0];
  TileMaxQueue<kSeg> tq(my_row < N ? tilemax + ((size_t)bh * N + my_row) * ktp : nullptr);
  // one tile: scores for both query blocks, optional masking, maxima
  auto tile = [&](int kt, auto masked) {
    float tmax[2];
    const char* kl = smem + (kt & 1) * kBK * KS;
    f32x16 acc[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) acc[qb][0] = acc[qb][1] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<E> a;
        ld8(a, reinterpret_cast<const E*>(kl + (32 * kb + c32) * KS) + 16 * c + 8 * h);
        mma(acc[0][kb], a, qf[0][c]);
        mma(acc[1][kb], a, qf[1][c]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (decltype(masked)::value) mask_rows_above(acc[qb], row_limit(kt * kBK, iq[qb], N, P.causal, h));
      // NaN-propagating maximum: v_maximum3_f32 with no canonicalising of the
      // MFMA results that fmaxf would need
      float tm = __builtin_elementwise_maximum(acc[qb][0][0], acc[qb][1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i)
        tm = __builtin_elementwise_maximum(tm, __builtin_elementwise_maximum(acc[qb][0][i], acc[qb][1][i]));
      m[qb] = fmaxf(m[qb], tm);
      tmax[qb] = tm;
    }
    // each row's maximum over the tile (lanes l and l^32 hold its two
    // halves); lane half h stores the value of query block h
    const float r0 = half_swap_max(tmax[0]);
    const float r1 = half_swap_max(tmax[1]);
    tq.push(half_bits_up((h ? r1 : r0) * P.scale));
    tq.tile_done(kt);
  };

  int kt = 0;
  for (; kt < kt_full; ++kt) {
    if (kt + 1 < kt_end) st.load(Kh, (kt + 1) * kBK, N);
    tile(kt, std::false_type{});
    if (kt + 1 < kt_end) st.store(smem + ((kt + 1) & 1) * kBK * KS, KS);
    __syncthreads();
  }
  for (; kt < kt_end; ++kt) {
    if (kt + 1 < kt_end) st.load(Kh, (kt + 1) * kBK, N);
    if (kt < kt_end_w) tile(kt, std::true_type{});
    if (kt + 1 < kt_end) st.store(smem + ((kt + 1) & 1) * kBK * KS, KS);
    __syncthreads();
  }
  tq.finish(max(kt_end_w, kt_full));
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float mm = fmaxf(m[qb], __shfl_xor(m[qb], 32));
    if (iq[qb] < N && h == 0) rowmax[(size_t)bh * N + iq[qb]] = mm * P.scale;
  }
}

// The same sweep for bf16 inputs on 16x16x32 MFMA: sixteen independent
// accumulators per wave (4 key blocks x 4 query blocks of 16) keep the matrix
// pipe fed without dependent-issue stalls.  Operand layout of
// v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16): A[l % 16][8g + j],
// B[8g + j][l % 16], C[4g + i][l % 16].  A = K rows, B = Q^T, so C is S^T and
// lane l holds, for query (l % 16) of each query block, keys 4g + i of each
// key block.
__device__ __forceinline__ f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
constexpr int kRowmaxTPS = 2;      // K tiles per barrier step (two steps of slots in LDS)
template <int D>
__global__ __launch_bounds__(kThreads) void k_rowmax16(const __bf16* __restrict__ Q,
                                                       const __bf16* __restrict__ K, Params P,
                                                       float* __restrict__ rowmax,
                                                       uint16_t* __restrict__ tilemax) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using DT = DirectTile<D>;
  constexpr int TPS = kRowmaxTPS;
  constexpr int KST = D / 32;      // contraction steps of 32
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int N = P.N;
  const int n_qt = (N + 255) / 256;
  // Causal query tile t holds 4 (t + 1) key tiles of work.  With pair_qt a
  // workgroup takes the pair (n_qt - 1 - t, t), so that every workgroup
  // sweeps the same number of tiles (the middle tile of an odd count runs
  // alone); otherwise one tile per workgroup, heaviest first.
  int bh, unit;
  map_tile(P.pair_qt ? (n_qt + 1) / 2 : n_qt, P.BH, P.causal && !P.pair_qt, bh, unit);
  const __bf16* Qh = Q + (size_t)bh * N * D;
  const __bf16* Kh = K + (size_t)bh * N * D;
  const DT dt(Kh, N, w, lane);
  const int ktp = tilemax_row(P.n_kt);
  constexpr int kSeg = D == 64 ? 1 : 4;

  auto sweep = [&](int qtile) {
    const int q0 = qtile * 256;
    const int wq0 = q0 + 64 * w;
    // B fragments: query wq0 + 16 b + c16, dimensions 32 ks + 8 g ... + 7
    bf16x8 qf[4][KST];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int qi = wq0 + 16 * b + c16;
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
        qf[b][ks] = qi < N ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)qi * D + 32 * ks + 8 * g)
                           : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    const int iq = wq0 + lane;       // the query whose maxima this lane keeps
    const int kt_end = P.causal ? (min(N - 1, q0 + 255) / kBK + 1) : P.n_kt;
    const int kt_end_w = wq0 >= N ? 0 : (P.causal ? (min(N - 1, wq0 + 63) / kBK + 1) : P.n_kt);
    const int kt_full = min(P.causal ? q0 / kBK : P.n_kt, N / kBK);

#pragma unroll
    for (int j = 0; j < TPS; ++j)
      if (j < kt_end) dt.issue(smem + j * DT::BYTES, j * kBK, w);

    TileMaxQueue<kSeg> tq(iq < N ? tilemax + ((size_t)bh * N + iq) * ktp : nullptr);
    float m = -INFINITY;

    auto tile = [&](int kt, auto masked) {
      const char* kl = smem + (kt % (2 * TPS)) * DT::BYTES;
      f32x4 acc[4][4];               // [query block][key block]
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[b][kb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(DT::at(kl, 16 * kb + c16, 4 * ks + g));
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[b][kb] = mma16(a, qf[b][ks], acc[b][kb]);
        }
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int qi = wq0 + 16 * b + c16;
          // last visible key of query qi, relative to this lane's first key
          const int lim = (qi >= N ? -1 : (P.causal ? min(qi, N - 1) : N - 1)) - kt * kBK - 4 * g;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kb + i > lim) acc[b][kb][i] = -INFINITY;
        }
      }
      float pm[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float t = __builtin_elementwise_maximum(acc[b][0][0], acc[b][0][1]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = (kb == 0 ? 2 : 0); i < 4; ++i) t = __builtin_elementwise_maximum(t, acc[b][kb][i]);
        pm[b] = t;
      }
      // Reduce over the four lane groups and scatter: group g keeps query
      // block g.  permlane32 swap pairs groups (0,2) and (1,3) for blocks
      // (0,2) and (1,3); permlane16 swap then pairs (0,1) and (2,3).
      const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[0]), __float_as_uint(pm[2]), false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[1]), __float_as_uint(pm[3]), false, false);
      const float a0 = __builtin_elementwise_maximum(__uint_as_float(s02[0]), __uint_as_float(s02[1]));
      const float a1 = __builtin_elementwise_maximum(__uint_as_float(s13[0]), __uint_as_float(s13[1]));
      const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
      const float tm = __builtin_elementwise_maximum(__uint_as_float(s01[0]), __uint_as_float(s01[1]));
      m = fmaxf(m, tm);
      tq.push(half_bits_up(tm * P.scale));
      tq.tile_done(kt);
    };

    // Step over TPS tiles: wait for them (issued one step earlier; this also
    // retires the tile-max stores), bare barrier (a full __syncthreads would
    // add a memory fence), issue the next step's tiles into the slots that
    // the previous step read, compute.
    for (int kt0 = 0; kt0 < kt_end; kt0 += TPS) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int j = 0; j < TPS; ++j) {
        const int kn = kt0 + TPS + j;
        if (kn < kt_end) dt.issue(smem + (kn % (2 * TPS)) * DT::BYTES, kn * kBK, w);
      }
#pragma unroll
      for (int j = 0; j < TPS; ++j) {
        const int kt = kt0 + j;
        if (kt < kt_full)
          tile(kt, std::false_type{});
        else if (kt < kt_end_w)
          tile(kt, std::true_type{});
      }
    }
    tq.finish(max(kt_end_w, kt_full));
    if (iq < N) rowmax[(size_t)bh * N + iq] = m * P.scale;
  };

  if (!P.pair_qt) {
    sweep(unit);
  } else {
    const int heavy = n_qt - 1 - unit;
    sweep(heavy);
    if (unit != heavy) {
      // every wave is done with the LDS slots before the next tile's first
      // loads land in them
      __builtin_amdgcn_s_barrier();
      sweep(unit);
    }
  }
}

// ---------------------------------------------------------- P V tile ---
// One key tile of O += P V for the 32 queries of a wave: scores from the
// staged K tile, p = [x - tau]_+^beta, then P V on MFMA with P as the B
// operand straight from the score accumulators.  bf16: V is a row-major tile
// (row stride VS) read down its columns; fp32: V^T columns [D][VS].
template <typename E, int D, int AK, bool M>
__device__ __forceinline__ void pv_tile(f32x16 (&oacc)[D / 32], const char* kl, const char* vl, int VS,
                                        const Frag<E> (&qf)[D / 16], int lane, int lim, float tau,
                                        const Params& P) {
  constexpr bool kTr = sizeof(E) == 2;
  constexpr int KS = row_stride<E, D>();
  const int h = lane >> 5, c32 = lane & 31;
  f32x16 acc[2];
  tile_scores<E, D>(acc, kl, KS, qf, lane, lim, std::integral_constant<bool, M>{});
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float t = clamp01(fmaf(acc[kb][j], P.scale, -tau));
      float p, u;
      Ent<AK>::pu(t, P.beta, p, u);
      acc[kb][j] = p;
    }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      Frag<E> pf;
      from_acc(pf, acc[kb], 8 * s);
      const int koff = 32 * kb + 16 * s + 4 * h;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        Frag<E> vf;
        if constexpr (kTr) {
          ld_col8(vf, vl, VS, koff, 32 * db, lane);
        } else {
          const E* vrow = reinterpret_cast<const E*>(vl + (32 * db + c32) * VS);
          ld4x2(vf, vrow + koff, vrow + koff + 8);
        }
        mma(oacc[db], vf, pf);
      }
    }
}

// Writes a wave's O accumulators for query iq (fp32 or bf16 out).
template <int D>
__device__ __forceinline__ void store_out(const f32x16 (&oacc)[D / 32], void* out, size_t row, int h,
                                          bool out_bf16) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * h;
      const size_t off = row * D + d0;
      const f32x4 o = f32x4{oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
      if (out_bf16) {
        const bf16x4 ob = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) + off) = ob;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = o;
      }
    }
}

// z^beta for z > 0 (0 otherwise), in deriv z^(beta-1): the power of the
// histogram's estimate for alpha other than 1.5 and 2 (float accuracy is
// ample for a start value).
template <int AK>
__device__ __forceinline__ float model_pow(float z, float beta, float& deriv) {
  if (!(z > 0.0f)) {
    deriv = 0.0f;
    return 0.0f;
  }
  if constexpr (AK == AK125) {   // beta = 4
    const float z2 = z * z;
    deriv = z2 * z;
    return z2 * z2;
  } else {
    const float l = log2f(z);
    deriv = exp2f((beta - 1.0f) * l);
    return exp2f(beta * l);
  }
}

// ------------------------------------------------------------- k_tau ---
// Per workgroup (128 queries, 32 per wave): bracket from the row maxima and
// the row's tile maxima, candidate key tiles, histogram initialisation,
// Halley / bisection sweeps over candidate tiles, tau, iteration counts and
// the block mask.  Dynamic LDS: K double buffer | histogram [128][BINS*2+2] u64 |
// list i16[kChunk] | wave bits u8[kChunk] | flags u8[kChunk] |
// candidate bits u32[4][n_words] | counter.
constexpr int kChunk = 512;    // key tiles listed at once

template <typename E, int D>
constexpr int tau_region_bytes(int bins) {
  // histogram [128][2 bins + 2] u64; for bf16 also the V double buffer of the
  // P V epilogue, which reuses it
  return sizeof(E) == 2 && 2 * kBK * row_stride<E, D>() > kBQW * (2 * bins + 2) * 8
             ? 2 * kBK * row_stride<E, D>()
             : kBQW * (2 * bins + 2) * 8;
}

template <typename E, int D, int AK, int BINS>
__global__ __launch_bounds__(kThreads) void k_tau(const E* __restrict__ Q, const E* __restrict__ K,
                                                  const E* __restrict__ V,
                                                  const float* __restrict__ rowmax,
                                                  const uint16_t* __restrict__ tilemax, Params P,
                                                  float* __restrict__ tau_out,
                                                  uint8_t* __restrict__ mask_out,
                                                  uint8_t* __restrict__ iters_out,
                                                  void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int KS = row_stride<E, D>();
  constexpr bool kFusePV = sizeof(E) == 2;   // bf16: P V runs here, after tau
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = P.N;
  int bh, qtile;
  map_tile((N + kBQW - 1) / kBQW, P.BH, P.causal, bh, qtile);
  const int q0 = qtile * kBQW;
  const int wq0 = q0 + kBQ * w;
  const int iq = wq0 + c32;
  const bool valid = iq < N;
  const bool wave_rows = wq0 < N;
  const int r32 = qtile * kWaves + w;
  const E* Qh = Q + (size_t)bh * N * D;
  const E* Kh = K + (size_t)bh * N * D;
  const bool dense = (P.flags & EA_FLAG_FORCE_DENSE) != 0;

  // histogram rows are padded by one bin so the 32 rows of a wave updating
  // the same bin index do not hit the same LDS bank
  constexpr int HROW = BINS * 2 + 2;
  const int n_words = (P.n_kt + 31) >> 5;
  char* kbuf = smem;                                                  // 2 x [64][KS]
  unsigned long long* hist = reinterpret_cast<unsigned long long*>(smem + 2 * kBK * KS);
  short* list = reinterpret_cast<short*>(smem + 2 * kBK * KS + tau_region_bytes<E, D>(BINS));
  uint8_t* wbits = reinterpret_cast<uint8_t*>(list + kChunk);
  uint8_t* flags = wbits + kChunk;
  uint32_t* cbits = reinterpret_cast<uint32_t*>(flags + kChunk);      // [4][n_words]
  int* counter = reinterpret_cast<int*>(cbits + kWaves * n_words);
  uint32_t* mbits = reinterpret_cast<uint32_t*>(counter + 16);        // [4][n_words] final mask

  const int wq_last = min(N - 1, wq0 + kBQ - 1);
  const int kt_end_w = !wave_rows ? 0 : (P.causal ? wq_last / kBK + 1 : P.n_kt);
  const int kt_end = P.causal ? (min(N - 1, q0 + kBQW - 1) / kBK + 1) : P.n_kt;
  const bool wave_has_tail = wq0 + kBQ > N;

  const int ktp = tilemax_row(P.n_kt);
  // this row's tile maxima; lane half h reads the groups of 8 tiles 2i + h
  const uint16_t* tmx = tilemax + ((size_t)bh * N + (valid ? iq : 0)) * ktp;
  // 2 kGB groups of 8 tiles (kGB per lane half) per batch
  constexpr int kGB = AK == AKGEN ? 4 : 8;
  auto load_groups = [&](int g0, u32x4 (&r)[kGB]) {
#pragma unroll
    for (int u = 0; u < kGB; ++u) {
      const int g = g0 + 2 * u + h;
      if (valid && g * 8 < kt_end_w)
        r[u] = *reinterpret_cast<const u32x4*>(tmx + g * 8);
      else
        r[u] = u32x4{0xFC00FC00u, 0xFC00FC00u, 0xFC00FC00u, 0xFC00FC00u};
    }
  };
  // the first batch is in flight together with the query fragments
  u32x4 pre[kGB];
  load_groups(0, pre);

  Frag<E> qf[D / 16];
  load_qfrags<E, D>(qf, Qh + (size_t)iq * D, valid, h);

  // ---- provable bracket [lo, hi]:  f(max x - 1) >= 0 >= f(max x - n^(1-alpha))
  const float xmax = valid ? rowmax[(size_t)bh * N + iq] : 0.0f;
  float lo = 0.0f, hi = 0.0f, tau = 0.0f;
  if (valid) {
    const double dl = (double)xmax - 1.0;
    lo = (float)dl;
    if ((double)lo > dl) lo = nextafterf(lo, -INFINITY);
    const double n = P.causal ? (double)(iq + 1) : (double)N;
    const double dh = (double)xmax - pow(n, 1.0 - (double)P.alpha);
    hi = (float)dh;
    if ((double)hi < dh) hi = nextafterf(hi, INFINITY);
    if (hi < lo) hi = lo;
  }
  bool conv = !valid;
  int iters = 0;
  const double beta = (double)P.beta;
  int* ncand = counter + 1;                                   // [4]
  // half bits of tile g*8 + j from a loaded group (-inf past the wave's end)
  auto group_half = [&](const u32x4& r, int g, int j) -> uint16_t {
    const uint32_t wrd = r[j >> 1];
    const uint16_t b = (uint16_t)((j & 1) ? (wrd >> 16) : (wrd & 0xFFFFu));
    return (g * 8 + j < kt_end_w) ? b : (uint16_t)0xFC00u;
  };

  // ---- candidate key tiles: bit kt of wave w is set when some row of the
  // wave has a tile maximum above its lower bracket end (tau >= lo, so no
  // other tile can hold a nonzero probability for the wave).  Returns the
  // workgroup's number of candidate wave-tiles, counted as if skipping were
  // on, so that every decision taken from it is the same either way.
  auto make_cand = [&](auto use_pre) -> int {
    __syncthreads();   // earlier readers of the bits and counts are done
    const float lim = valid ? lo - 4.0f * FLT_EPSILON * fmaxf(1.0f, fabsf(lo)) : INFINITY;
    int total = 0;
    // batch of 16 kGB tiles = kGB / 2 words; group g = 2i + h covers tiles 8g..8g+7
    for (int g0 = 0; g0 * 8 < kt_end; g0 += 2 * kGB) {   // later tiles are never listed
      u32x4 r[kGB];
      if (decltype(use_pre)::value && g0 == 0) {
#pragma unroll
        for (int u = 0; u < kGB; ++u) r[u] = pre[u];
      } else {
        load_groups(g0, r);
      }
      // this row's candidate bits, 8 per group, then OR over the half's rows
      uint32_t pl[kGB / 4];
#pragma unroll
      for (int q = 0; q < kGB / 4; ++q) pl[q] = 0u;
#pragma unroll
      for (int u = 0; u < kGB; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (half_up_value(group_half(r[u], g0 + 2 * u + h, j)) > lim) pl[u >> 2] |= 1u << (8 * (u & 3) + j);
#pragma unroll
      for (int q = 0; q < kGB / 4; ++q) {
        const unsigned long long hv = half_or_dpp(pl[q]);
        const uint32_t h0 = (uint32_t)hv, h1 = (uint32_t)(hv >> 32);
        // word k of this batch: groups g0+4k (half 0, u=2k), g0+4k+1 (half 1,
        // u=2k), g0+4k+2 (half 0, u=2k+1), g0+4k+3 (half 1, u=2k+1)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int sh = 16 * kk;
          const uint32_t real = ((h0 >> sh) & 0xFFu) | (((h1 >> sh) & 0xFFu) << 8) |
                                (((h0 >> (sh + 8)) & 0xFFu) << 16) | (((h1 >> (sh + 8)) & 0xFFu) << 24);
          const int wd = (g0 * 8 >> 5) + 2 * q + kk;
          const int nv = min(max(kt_end_w - 32 * wd, 0), 32);
          const uint32_t vis = nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u);
          total += __popc(real);
          if (lane == 0 && wd < n_words) cbits[w * n_words + wd] = dense ? vis : real;
        }
      }
    }
    if (lane == 0) ncand[w] = total;
    __syncthreads();
    return ncand[0] + ncand[1] + ncand[2] + ncand[3];
  };
  auto cand = [&](int ww, int kt) -> bool { return (cbits[ww * n_words + (kt >> 5)] >> (kt & 31)) & 1u; };
  // visible wave-tiles of the workgroup (the same for every thread)
  int vis_total = 0;
  for (int ww = 0; ww < kWaves; ++ww) {
    const int wq = q0 + kBQ * ww;
    if (wq < N) vis_total += P.causal ? min(N - 1, wq + kBQ - 1) / kBK + 1 : P.n_kt;
  }
  // Pruning pays for its extra passes over the tile maxima (a few memory
  // round trips) only when the bracket [max x - 1, ...] leaves many tiles
  // standing, both in number and as a share of the visible ones.
  const int n_cand0 = make_cand(std::true_type{});
  const bool wide = n_cand0 >= 64 && n_cand0 * 8 > vis_total;

  // ---- lower bracket end from the row's tile maxima M_t.  Every tile holds
  // its maximum element, so g(t) = sum_t [M_t - t]_+^beta - 1 <= f(t): g's root
  // is a valid lower bound on tau, and a tight one when many tiles reach near
  // the row maximum.  Halley-bisection on g over lower bounds of the tile
  // maxima (the two lane halves take alternate tiles); the largest point with
  // g >= 0 is kept.
  if (wide && P.mode != EA_TAU_BISECT) {
    float glo = lo, ghi = hi, tg = lo;
    for (int it = 0; it < 3; ++it) {
      float G0 = 0, G1 = 0, G2 = 0, gc = 0;
      for (int g0 = 0; g0 * 8 < kt_end_w; g0 += 2 * kGB) {
        u32x4 r[kGB];
        load_groups(g0, r);
#pragma unroll
        for (int u = 0; u < kGB; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            Ent<AK>::sweep(clamp01(half_down_value(group_half(r[u], g0 + 2 * u + h, j)) - tg), P.beta,
                           G0, G1, G2, gc);
      }
      G0 += __shfl_xor(G0, 32);
      G1 += __shfl_xor(G1, 32);
      G2 += __shfl_xor(G2, 32);
      const double g = (double)G0 - 1.0;
      if (g >= 0.0) glo = tg; else ghi = tg;
      const double ulp = (double)FLT_EPSILON * fmax(1.0, fabs((double)tg));
      const double gp = -beta * (double)G1;
      const double gpp = (AK == AK20) ? 0.0 : beta * (beta - 1.0) * (double)G2;
      const double th = (double)tg - 2.0 * g * gp / (2.0 * gp * gp - g * gpp);
      float nt = (th > (double)glo && th < (double)ghi) ? (float)th : glo + 0.5f * (ghi - glo);
      if (!(nt > glo && nt < ghi) || fabs(g) <= 2.0 * fabs(gp) * ulp || ghi - glo <= 4.0f * (float)ulp) break;
      tg = nt;
    }
    glo -= 4.0f * FLT_EPSILON * fmaxf(1.0f, fabsf(glo));
    if (valid && glo > lo) lo = fminf(glo, hi);
    make_cand(std::false_type{});
  }

  // ---- histogram initialisation (AdaSplash-2)
  if (P.mode == EA_TAU_HIST_HALLEY) {
    for (int e = threadIdx.x; e < kBQW * HROW; e += kThreads) hist[e] = 0ull;
    unsigned long long* hr = hist + (size_t)(kBQ * w + c32) * HROW;
    // bins split [lo, hi]; moments are kept in units of 2^-24 of y = x - lo <= 1
    const float width = valid ? fmaxf(hi - lo, 1e-30f) : 1.0f;
    const float bin_scale = (float)BINS / width;
    for (int base = 0; base < kt_end; base += kChunk) {
      const int n = build_list(base, min(kChunk, kt_end - base), cand, list, wbits, flags, counter);
      RowTiles<E, D, kBK> st(Kh, N, w, lane);
      if (n > 0) {
        st.fetch(kbuf, (base + list[0]) * kBK);
        st.commit(kbuf);
      }
      __syncthreads();
      for (int i = 0; i < n; ++i) {
        const int kt = base + list[i];
        if (i + 1 < n) st.fetch(kbuf + ((i + 1) & 1) * kBK * KS, (base + list[i + 1]) * kBK);
        if ((wbits[i] >> w) & 1) {
          auto body = [&](auto masked) {
            f32x16 acc[2];
            tile_scores<E, D>(acc, kbuf + (i & 1) * kBK * KS, KS, qf, lane,
                              row_limit(kt * kBK, iq, N, P.causal, h), masked);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                const float y = fmaf(acc[kb][j], P.scale, -lo);
                if (y > 0.0f) {
                  const unsigned Y = (unsigned)(fminf(y, 1.0f) * 16777216.0f);
                  const int b = min((int)(y * bin_scale), BINS - 1);
                  atomicAdd(&hr[2 * b], (1ull << 40) + (unsigned long long)Y);
                  atomicAdd(&hr[2 * b + 1], (unsigned long long)Y * (unsigned long long)Y);
                }
              }
          };
          if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
            body(std::true_type{});
          else
            body(std::false_type{});
        }
        if (i + 1 < n) st.commit(kbuf + ((i + 1) & 1) * kBK * KS);
        __syncthreads();
      }
    }
    if (valid) {
      const double inv24 = 1.0 / 16777216.0, inv48 = inv24 * inv24;
      const double bw = (double)width / BINS;     // bin width in y = x - lo
      const bool exact = (AK == AK15 || AK == AK20);
      double C = 0, S1 = 0, S2 = 0;       // moments of the bins above the edge under test
      double f_hi = -1.0;                  // f at the upper edge of the bin under test
      int bstar = 0;
      double f_lo = 0, cstar = 0, Cs = 0, S1s = 0, S2s = 0;
      // Other alpha (estimate only): the elements of every bin b0.. stand
      // half at mu - sd and half at mu + sd of their bin, which keeps the
      // bin's count, sum and sum of squares.  Returns f of that model at t
      // (float: a start value needs no more) and its derivative in df.
      auto model_f = [&](int b0, float t, float& df) -> float {
        float fv = -1.0f;
        df = 0.0f;
        for (int bb = b0; bb < BINS; ++bb) {
          const unsigned long long g1 = hr[2 * bb], g2 = hr[2 * bb + 1];
          const float cc = (float)(g1 >> 40);
          if (cc > 0.0f) {
            const float mu = (float)((double)(g1 & ((1ull << 40) - 1ull)) * inv24) / cc;
            const float sd = sqrtf(fmaxf((float)((double)g2 * inv48) / cc - mu * mu, 0.0f));
            float da, db;
            const float va = model_pow<AK>(mu + sd - t, P.beta, da);
            const float vb = model_pow<AK>(mu - sd - t, P.beta, db);
            fv += 0.5f * cc * (va + vb);
            df -= 0.5f * cc * P.beta * (da + db);
          }
        }
        return fv;
      };
      for (int b = exact ? BINS - 1 : -1; b >= 0; --b) {   // the exact edge values
        const unsigned long long h1 = hr[2 * b], h2 = hr[2 * b + 1];
        const double cb = (double)(h1 >> 40);
        const double s1 = (double)(h1 & ((1ull << 40) - 1ull)) * inv24;
        const double s2 = (double)h2 * inv48;
        const double e = (double)b * bw;
        const double Cn = C + cb, S1n = S1 + s1, S2n = S2 + s2;
        double f;
        if (AK == AK15) {
          f = S2n - 2.0 * e * S1n + e * e * Cn - 1.0;      // exact at the edge
        } else {
          f = S1n - e * Cn - 1.0;                          // AK20: exact at the edge
        }
        if (f >= 0.0 || b == 0) {
          bstar = b;
          f_lo = f;
          cstar = cb;
          Cs = C;
          S1s = S1;
          S2s = S2;
          break;
        }
        f_hi = f;
        C = Cn;
        S1 = S1n;
        S2 = S2n;
      }
      if (!exact) {
        // the model decreases in t: tau's bin by bisection over the edges
        int blo = 0, bhi = BINS;
        while (bhi - blo > 1) {
          const int mid = (blo + bhi) >> 1;
          float df;
          if (model_f(mid, (float)(mid * bw), df) >= 0.0f) blo = mid; else bhi = mid;
        }
        bstar = blo;
      }
      const double eb = (double)bstar * bw, eb1 = (double)(bstar + 1) * bw;
      double t0 = -1.0;
      if (!exact) {
        // Newton on the model from the bin's lower edge: the model is convex
        // and decreasing, so the steps rise monotonically to its root
        float t = (float)eb;
        const float tmax = (float)eb1, dt = 1e-6f * (float)bw;
        for (int it2 = 0; it2 < 8; ++it2) {
          float df;
          const float fv = model_f(bstar, t, df);
          if (!(fv > 0.0f) || !(df < 0.0f)) break;
          const float tn = fminf(t - fv / df, tmax);
          if (!(tn > t + dt)) {
            t = fmaxf(t, tn);
            break;
          }
          t = tn;
        }
        t0 = (double)t;
      }
      if (exact && cstar == 0.0 && Cs > 0.0) {
        // the tau bin is empty: the support is exactly the bins above it
        if (AK == AK15) {
          const double disc = S1s * S1s - Cs * (S2s - 1.0);
          if (disc >= 0.0) t0 = (S1s - sqrt(disc)) / Cs;
        } else {
          t0 = (S1s - 1.0) / Cs;
        }
        if (!(t0 >= eb && t0 <= eb1)) t0 = -1.0;
      }
      if (exact && t0 < 0.0 && cstar > 0.0) {
        // tau's bin holds elements: f is exact for the bins above it, and the
        // bin's own cstar elements are replaced by cstar/2 at each of mu - sd
        // and mu + sd, which keeps their count, sum and sum of squares.  The
        // model equals f at both edges; its root is the start.
        const unsigned long long g1 = hr[2 * bstar], g2 = hr[2 * bstar + 1];
        const double s1b = (double)(g1 & ((1ull << 40) - 1ull)) * inv24;
        const double s2b = (double)g2 * inv48;
        const double mu = s1b / cstar;
        const double sd = sqrt(fmax(s2b / cstar - mu * mu, 0.0));
        const double p2 = mu + sd;
        const double q1 = fmin(fmax(mu - sd, eb), eb1), q2 = fmin(fmax(p2, eb), eb1);
        // segments [eb, q1], [q1, q2], [q2, eb1]: moments of what lies above tau
        const double segA[3] = {Cs + cstar, Cs + 0.5 * cstar, Cs};
        const double segB[3] = {S1s + s1b, S1s + 0.5 * cstar * p2, S1s};
        const double segS[3] = {S2s + s2b, S2s + 0.5 * cstar * p2 * p2, S2s};
        const double segR[3] = {q1, q2, eb1};
        double a0 = eb;
        for (int sg = 0; sg < 3; ++sg) {
          const double A = segA[sg], B = segB[sg], S = segS[sg], a1 = segR[sg];
          const double fr = (AK == AK15) ? S - 2.0 * a1 * B + a1 * a1 * A - 1.0 : B - a1 * A - 1.0;
          if (a1 > a0 && fr <= 0.0) {
            double t = -1.0;
            if (AK == AK15) {
              const double disc = B * B - A * (S - 1.0);
              if (A > 0.0 && disc >= 0.0) t = (B - sqrt(disc)) / A;
            } else if (A > 0.0) {
              t = (B - 1.0) / A;
            }
            if (t >= 0.0) t0 = fmin(fmax(t, a0), a1);
            break;
          }
          a0 = fmax(a0, a1);
        }
      }
      if (t0 < 0.0) {
        const double den = f_lo - f_hi;
        t0 = den > 0.0 ? eb + (eb1 - eb) * (f_lo / den) : 0.5 * (eb + eb1);
      }
      const float t0x = (float)((double)lo + t0);
      if (exact) {
        const float margin = fmaxf(1.0f, fabsf(xmax)) * 5e-7f + 1e-6f;
        const float nlo = (float)((double)lo + eb) - margin;
        const float nhi = (float)((double)lo + eb1) + margin;
        if (nlo > lo) lo = nlo;
        if (nhi < hi) hi = nhi;
      }
      tau = fminf(fmaxf(t0x, lo), hi);
    }
    // the histogram narrowed lo to tau's bin: prune the candidates again
    if (wide && (AK == AK15 || AK == AK20)) make_cand(std::false_type{});
  } else if (P.mode == EA_TAU_HALLEY_BISECT) {
    tau = lo;
  } else {
    tau = 0.5f * (lo + hi);
  }

  // ---- refinement sweeps (Halley-bisection or bisection) over candidate tiles
  uint8_t* mrow = mask_out + ((size_t)bh * P.n_q32 + (size_t)r32) * P.n_kt;
  if (wave_rows) {
    for (int kt = lane; kt < P.n_kt; kt += kWave) mrow[kt] = (dense && kt < kt_end_w) ? 1 : 0;
  }
  if constexpr (kFusePV) {
    // the same mask as bits in LDS for the P V epilogue
    for (int e = lane; e < n_words; e += kWave) {
      const int nv = min(max(kt_end_w - 32 * e, 0), 32);
      mbits[w * n_words + e] = dense ? (nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u)) : 0u;
    }
  }
  const int max_iters = P.max_iters;
  // The candidate tiles do not change between refinement sweeps.  When the
  // workgroup's fit beside the K double buffer in the histogram's space (dead
  // from here), they are copied once and every sweep reads them in place: no
  // list rebuild, copy or barrier per tile.
  constexpr int kResident = 2 + tau_region_bytes<E, D>(BINS) / (kBK * KS);
  auto slot = [&](int i) -> char* {
    return i < 2 ? kbuf + i * kBK * KS : reinterpret_cast<char*>(hist) + (i - 2) * kBK * KS;
  };
  int n_res = -1;   // resident tile count, or -1: the sweeps stream their tiles
  if (kt_end <= kChunk) {
    const int n = build_list(0, kt_end, cand, list, wbits, flags, counter);
    if (n <= kResident) {
      RowTiles<E, D, kBK> st(Kh, N, w, lane);
      for (int i = 0; i < n; ++i) {
        st.fetch(slot(i), list[i] * kBK);
        st.commit(slot(i));
      }
      __syncthreads();
      n_res = n;
    }
  }
  for (int sweep = 0; sweep <= max_iters + 1; ++sweep) {
    const bool wave_busy = __ballot(!conv) != 0ull;
    if (!__syncthreads_or(wave_busy ? 1 : 0)) break;
    if (kFusePV && wave_busy && !dense) {
      // this sweep rewrites the wave's mask
      for (int e = lane; e < n_words; e += kWave) mbits[w * n_words + e] = 0u;
    }
    float F0 = 0, F1 = 0, F2 = 0, cnt = 0;
    // f, f', f'' terms of key tile kt (staged at kl) and its mask bits
    auto sweep_tile = [&](int kt, const char* kl) {
      auto body = [&](auto masked) {
        f32x16 acc[2];
        tile_scores<E, D>(acc, kl, KS, qf, lane, row_limit(kt * kBK, iq, N, P.causal, h), masked);
        const float before = Ent<AK>::count(F0, F1, F2, cnt);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float t = clamp01(fmaf(acc[kb][j], P.scale, -tau));
            Ent<AK>::sweep(t, P.beta, F0, F1, F2, cnt);
          }
        if (!dense) {
          const bool any = __ballot(Ent<AK>::count(F0, F1, F2, cnt) > before) != 0ull;
          if (lane == (kt & (kWave - 1))) mrow[kt] = any ? 1 : 0;   // same lane as the zero fill
          if (kFusePV && any && lane == 0) atomicOr(&mbits[w * n_words + (kt >> 5)], 1u << (kt & 31));
        }
      };
      if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
        body(std::true_type{});
      else
        body(std::false_type{});
    };
    if (n_res >= 0) {
      for (int i = 0; i < n_res; ++i)
        if (wave_busy && ((wbits[i] >> w) & 1)) sweep_tile(list[i], slot(i));
    } else {
      for (int base = 0; base < kt_end; base += kChunk) {
        const int n = build_list(base, min(kChunk, kt_end - base), cand, list, wbits, flags, counter);
        RowTiles<E, D, kBK> st(Kh, N, w, lane);
        if (n > 0) {
          st.fetch(kbuf, (base + list[0]) * kBK);
          st.commit(kbuf);
        }
        __syncthreads();
        for (int i = 0; i < n; ++i) {
          if (i + 1 < n) st.fetch(kbuf + ((i + 1) & 1) * kBK * KS, (base + list[i + 1]) * kBK);
          if (wave_busy && ((wbits[i] >> w) & 1)) sweep_tile(base + list[i], kbuf + (i & 1) * kBK * KS);
          if (i + 1 < n) st.commit(kbuf + ((i + 1) & 1) * kBK * KS);
          __syncthreads();
        }
      }
    }
    F0 += __shfl_xor(F0, 32);
    F1 += __shfl_xor(F1, 32);
    F2 += __shfl_xor(F2, 32);
    if (!conv) {
      ++iters;
      const double f = (double)F0 - 1.0;
      // tau is a float: one ulp of tau moves f by about |f'| ulp, so |f| below
      // that granularity (or a Halley step below two ulps) is machine precision.
      const double ulp = (double)FLT_EPSILON * fmax(1.0, fabs((double)tau));
      const double fp = -beta * (double)F1;
      const bool bisect = P.mode == EA_TAU_BISECT;
      if (fabs(f) <= (double)P.tol + (bisect ? 0.0 : 2.0 * fabs(fp) * ulp)) {
        conv = true;
      } else {
        if (f > 0.0) lo = tau; else hi = tau;
        const float wtol = bisect ? 1e-6f * fmaxf(1.0f, fabsf(tau)) : 4.0f * (float)ulp;
        if (hi - lo <= wtol || iters >= max_iters) {
          conv = true;
        } else {
          double next = 0.5 * ((double)lo + (double)hi);
          if (!bisect) {
            const double fpp = (AK == AK20) ? 0.0 : beta * (beta - 1.0) * (double)F2;
            const double den = 2.0 * fp * fp - f * fpp;
            const double th = (double)tau - 2.0 * f * fp / den;
            if (fabs(th - (double)tau) <= 2.0 * ulp) {
              conv = true;                        // converged: keep the evaluated tau
            } else if (th > (double)lo && th < (double)hi) {
              next = th;
            }
          }
          if (!conv) {
            float nt = (float)next;
            if (!(nt > lo && nt < hi)) nt = lo + 0.5f * (hi - lo);
            if (!(nt > lo && nt < hi)) conv = true;   // bracket exhausted in float
            else tau = nt;
          }
        }
      }
    }
  }

  if (valid && h == 0) {
    tau_out[(size_t)bh * N + iq] = tau;
    if (iters_out) iters_out[(size_t)bh * N + iq] = (uint8_t)min(iters, 255);
  }

  // ---- P V over the active tiles of the final mask (bf16).  Q is still in
  // registers, tau in a register and the mask in LDS; V tiles take the
  // histogram's place.
  if constexpr (kFusePV) {
    __syncthreads();   // every wave's final mask bits (and the histogram is dead)
    char* vbuf = reinterpret_cast<char*>(hist);                       // 2 x [64][KS]
    const E* Vh = V + (size_t)bh * N * D;
    const float ptau = valid ? tau : INFINITY;
    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    auto active = [&](int ww, int kt) -> bool { return (mbits[ww * n_words + (kt >> 5)] >> (kt & 31)) & 1u; };
    RowTiles<E, D, kBK> sk(Kh, N, w, lane), sv(Vh, N, w, lane);
    for (int base = 0; base < kt_end; base += kChunk) {
      const int n = build_list(base, min(kChunk, kt_end - base), active, list, wbits, flags, counter);
      if (n > 0) {
        sk.fetch(kbuf, (base + list[0]) * kBK);
        sv.fetch(vbuf, (base + list[0]) * kBK);
        sk.commit(kbuf);
        sv.commit(vbuf);
      }
      __syncthreads();
      for (int i = 0; i < n; ++i) {
        const int kt = base + list[i];
        const int nb = (i + 1) & 1;
        if (i + 1 < n) {
          sk.fetch(kbuf + nb * kBK * KS, (base + list[i + 1]) * kBK);
          sv.fetch(vbuf + nb * kBK * KS, (base + list[i + 1]) * kBK);
        }
        if ((wbits[i] >> w) & 1) {
          const char* kl = kbuf + (i & 1) * kBK * KS;
          const char* vl = vbuf + (i & 1) * kBK * KS;
          const int lim = row_limit(kt * kBK, iq, N, P.causal, h);
          if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
            pv_tile<E, D, AK, true>(oacc, kl, vl, KS, qf, lane, lim, ptau, P);
          else
            pv_tile<E, D, AK, false>(oacc, kl, vl, KS, qf, lane, lim, ptau, P);
        }
        if (i + 1 < n) {
          sk.commit(kbuf + nb * kBK * KS);
          sv.commit(vbuf + nb * kBK * KS);
        }
        __syncthreads();
      }
    }
    if (valid) store_out<D>(oacc, out, (size_t)bh * N + iq, h, P.out_bf16 != 0);
  }
}

// -------------------------------------------------------------- k_pv ---
// Per workgroup (128 queries): O = P V over the active key tiles of the
// block mask.  bf16: V tiles are staged as rows and read down their columns with
// transposed LDS reads; fp32: Vsrc is a V^T copy [BH][D][Np].
template <typename E, int D, int AK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 4 && D == 128 ? 1 : 2, 2))) void k_pv(const E* __restrict__ Q, const E* __restrict__ K,
                                                 const E* __restrict__ Vsrc,
                                                 const float* __restrict__ tau_in,
                                                 const uint8_t* __restrict__ mask, Params P,
                                                 void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool kTr = sizeof(E) == 2;
  constexpr int KS = row_stride<E, D>();
  constexpr int VS = kTr ? KS : kBK * (int)sizeof(E) + 16;
  constexpr int VT = kTr ? kBK * KS : D * VS;      // bytes of one staged V tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = P.N;
  int bh, qtile;
  map_tile((N + kBQW - 1) / kBQW, P.BH, P.causal, bh, qtile);
  const int wq0 = qtile * kBQW + kBQ * w;
  const int iq = wq0 + c32;
  const bool valid = iq < N;
  const E* Qh = Q + (size_t)bh * N * D;
  const E* Kh = K + (size_t)bh * N * D;
  const E* Vh = kTr ? Vsrc + (size_t)bh * N * D : Vsrc + (size_t)bh * D * P.Np;

  char* kbuf = smem;                                 // 2 x [64][KS]
  char* vbuf = kbuf + 2 * kBK * KS;                  // 2 x V tile
  short* list = reinterpret_cast<short*>(vbuf + 2 * VT);
  uint8_t* wbits = reinterpret_cast<uint8_t*>(list + kChunk);
  uint8_t* flags = wbits + kChunk;
  int* counter = reinterpret_cast<int*>(flags + kChunk);

  Frag<E> qf[D / 16];
  load_qfrags<E, D>(qf, Qh + (size_t)iq * D, valid, h);
  const float tau = valid ? tau_in[(size_t)bh * N + iq] : INFINITY;
  const bool wave_has_tail = wq0 + kBQ > N;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  const size_t mrow0 = (size_t)bh * P.n_q32 + (size_t)qtile * kWaves;
  auto active = [&](int ww, int kt) -> bool {
    return (qtile * kWaves + ww) < P.n_q32 && mask[(mrow0 + ww) * P.n_kt + kt] != 0;
  };
  RowTiles<E, D, kBK> sk(Kh, N, w, lane);
  RowTiles<E, D, kBK> svr(Vh, N, w, lane);   // bf16 V rows
  ColStage<E, D, kBK> svc;                    // fp32 V^T columns
  auto load = [&](int k0, int b) {
    sk.fetch(kbuf + b * kBK * KS, k0);
    if constexpr (kTr) svr.fetch(vbuf + b * VT, k0);
    else svc.load(Vh, P.Np, k0);
  };
  auto store = [&](int b) {
    sk.commit(kbuf + b * kBK * KS);
    if constexpr (kTr) svr.commit(vbuf + b * VT);
    else svc.store(vbuf + b * VT, VS);
  };
  for (int base = 0; base < P.n_kt; base += kChunk) {
    const int n = build_list(base, min(kChunk, P.n_kt - base), active, list, wbits, flags, counter);
    if (n > 0) {
      load((base + list[0]) * kBK, 0);
      store(0);
    }
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const int kt = base + list[i];
      if (i + 1 < n) load((base + list[i + 1]) * kBK, (i + 1) & 1);
      if ((wbits[i] >> w) & 1) {
        const char* kl = kbuf + (i & 1) * kBK * KS;
        const char* vl = vbuf + (i & 1) * VT;
        const int lim = row_limit(kt * kBK, iq, N, P.causal, h);
        if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
          pv_tile<E, D, AK, true>(oacc, kl, vl, VS, qf, lane, lim, tau, P);
        else
          pv_tile<E, D, AK, false>(oacc, kl, vl, VS, qf, lane, lim, tau, P);
      }
      if (i + 1 < n) store((i + 1) & 1);
      __syncthreads();
    }
  }
  if (valid) store_out<D>(oacc, out, (size_t)bh * N + iq, h, P.out_bf16 != 0);
}

// --------------------------------------------------------- transposes ---
// [BH][N][D] -> [BH][D][Np], zero for n in [N, Np).
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E* __restrict__ in, E* __restrict__ outp,
                                                   int N, int D, int Np) {
  __shared__ E t[64][65];
  const E* src = in + (size_t)blockIdx.z * N * D;
  E* dst = outp + (size_t)blockIdx.z * D * Np;
  const int n0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    int r = e >> 6, c = e & 63;
    int n = n0 + r;
    t[r][c] = n < N ? src[(size_t)n * D + d0 + c] : (E)0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    int r = e >> 6, c = e & 63;
    dst[(size_t)(d0 + r) * Np + n0 + c] = t[c][r];
  }
}

// ---------------------------------------------------------- k_bwd_dq ---
// Per workgroup (128 queries), two passes over the active key tiles:
//  1. delta_i = sum_j u_ij dP_ij / sum_j u_ij (fp32, exact weights), written
//     out for the dK/dV kernel;
//  2. dQ = dS K / sqrt(d) with dS^T = U (dP^T - delta),
// where dP^T = V dO^T, all in the S^T layout.  bf16 reads the dQ operand
// down the columns of the staged K tile; fp32 stages K^T too.
template <typename E, int D, int AK, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 && (D == 128 || AK == AK15) ? 2 : 1, 2))) void k_bwd_dq(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const E* __restrict__ dO, const E* __restrict__ Kt, const float* __restrict__ tau_in,
    const uint8_t* __restrict__ mask, Params P, float* __restrict__ delta_out,
    uint8_t* __restrict__ maskT, void* __restrict__ dq) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool kTr = sizeof(E) == 2;
  constexpr int KS = row_stride<E, D>();
  constexpr int VS = kBK * (int)sizeof(E) + 16;
  constexpr int TT = kTr ? 0 : D * VS;              // bytes of one staged K^T tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = P.N;
  int bh, qtile;
  map_tile((N + kBQW - 1) / kBQW, P.BH, P.causal, bh, qtile);
  const int wq0 = qtile * kBQW + kBQ * w;
  const int iq = wq0 + c32;
  const bool valid = iq < N;
  const size_t hoff = (size_t)bh * N * D;
  const E* Kth = kTr ? nullptr : Kt + (size_t)bh * D * P.Np;

  // NB = 2: double-buffered tiles; NB = 1 when two copies exceed the LDS
  char* kbuf = smem;                                 // NB x [64][KS]
  char* vbuf = kbuf + NB * kBK * KS;                 // NB x [64][KS]
  char* tbuf = vbuf + NB * kBK * KS;                 // NB x [D][VS] (fp32 only)
  short* list = reinterpret_cast<short*>(tbuf + NB * TT);
  uint8_t* wbits = reinterpret_cast<uint8_t*>(list + kChunk);
  uint8_t* flags = wbits + kChunk;
  int* counter = reinterpret_cast<int*>(flags + kChunk);

  Frag<E> qf[D / 16], of[D / 16];
  load_qfrags<E, D>(qf, Q + hoff + (size_t)iq * D, valid, h);
  load_qfrags<E, D>(of, dO + hoff + (size_t)iq * D, valid, h);
  const float tau = valid ? tau_in[(size_t)bh * N + iq] : INFINITY;
  const bool wave_has_tail = wq0 + kBQ > N;

  f32x16 gacc[D / 32];                               // dQ, live in the second pass only
  float num = 0.0f, den = 0.0f, dlt = 0.0f;

  const size_t mrow0 = (size_t)bh * P.n_q32 + (size_t)qtile * kWaves;
  auto active = [&](int ww, int kt) -> bool {
    return (qtile * kWaves + ww) < P.n_q32 && mask[(mrow0 + ww) * P.n_kt + kt] != 0;
  };
  RowTiles<E, D, kBK> sk(K + hoff, N, w, lane), sv(V + hoff, N, w, lane);
  ColStage<E, D, kBK> st;
  // With one list chunk (n_kt <= kChunk) both passes walk the same list: it
  // is built once, and the first tile of pass 2 is fetched during the last
  // tile of pass 1.  Buffer parity then continues across the passes.
  const bool single = P.n_kt <= kChunk;
  int n_first = 0;
  // The two passes are unrolled and dQ is zeroed at the start of the second,
  // so its accumulators are not live during the first: 29 VGPRs spill at two
  // waves per SIMD (d = 128 bf16) instead of 73, and fewer scratch reloads
  // stall the next tile's copy.
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) gacc[db] = f32x16{};
    }
    auto load = [&](int ps, int k0, int b) {
      sk.fetch(kbuf + b * kBK * KS, k0);
      sv.fetch(vbuf + b * kBK * KS, k0);
      if constexpr (!kTr) {
        if (ps == 1) st.load(Kth, P.Np, k0);
      }
    };
    auto store = [&](int ps, int b) {
      sk.commit(kbuf + b * kBK * KS);
      sv.commit(vbuf + b * kBK * KS);
      if constexpr (!kTr) {
        if (ps == 1) st.store(tbuf + b * TT, VS);
      }
    };
    const bool reuse = single && pass == 1;          // list and first tile are ready
    const bool hand_over = single && pass == 0;      // fetch pass 2's first tile at the end
    for (int base = 0; base < P.n_kt; base += kChunk) {
      const int n = reuse ? n_first
                          : build_list(base, min(kChunk, P.n_kt - base), active, list, wbits, flags, counter);
      if (hand_over) n_first = n;
      const int s0 = reuse ? n_first : 0;            // step index of this pass's first tile
      if (n > 0 && !reuse) {
        load(pass, (base + list[0]) * kBK, 0);
        store(pass, 0);
      }
      __syncthreads();
      for (int i = 0; i < n; ++i) {
        const int kt = base + list[i];
        const int nb = NB == 2 ? ((s0 + i + 1) & 1) : 0;
        const bool next = i + 1 < n || hand_over;
        if (i + 1 < n)
          load(pass, (base + list[i + 1]) * kBK, nb);
        else if (hand_over)
          load(1, (base + list[0]) * kBK, nb);
        if ((wbits[i] >> w) & 1) {
          const int buf = NB == 2 ? ((s0 + i) & 1) : 0;
          const char* kl = kbuf + buf * kBK * KS;
          auto body = [&](auto masked) {
            // the tile in two 32-key halves: S and dP of one half (32 VGPRs) are
            // live at a time, which keeps the kernel's spills (and with them the
            // scratch reloads that wait for the next tile's copy) down
            const char* vl = vbuf + buf * kBK * KS;
            const char* tl = tbuf + buf * TT;
            const int lim = row_limit(kt * kBK, iq, N, P.causal, h);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              f32x16 sacc, pacc;
              scores_T_half2<E, D>(sacc, pacc, kl, vl, KS, kb, qf, of, lane);
              if constexpr (decltype(masked)::value) mask_half_rows_above(sacc, kb, lim);
              if (pass == 0) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                  const float t = clamp01(fmaf(sacc[j], P.scale, -tau));
                  float p, u;
                  Ent<AK>::pu(t, P.beta, p, u);
                  num = fmaf(u, pacc[j], num);
                  den += u;
                }
              } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                  const float t = clamp01(fmaf(sacc[j], P.scale, -tau));
                  float p, u;
                  Ent<AK>::pu(t, P.beta, p, u);
                  sacc[j] = u * (pacc[j] - dlt);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                  // dQ = sum_j dS_ij k_j cancels strongly when the supporting keys are
                  // nearly parallel (sum_j dS_ij = 0): dS goes in as a hi/lo bf16 pair.
                  Frag<E> sf, sl;
                  split_acc(sf, sl, sacc, 8 * s);
                  const int koff = 32 * kb + 16 * s + 4 * h;
#pragma unroll
                  for (int db = 0; db < D / 32; ++db) {
                    Frag<E> kf;
                    if constexpr (kTr) {
                      ld_col8(kf, kl, KS, koff, 32 * db, lane);
                    } else {
                      const E* krow = reinterpret_cast<const E*>(tl + (32 * db + c32) * VS);
                      ld4x2(kf, krow + koff, krow + koff + 8);
                    }
                    mma(gacc[db], kf, sf);
                    if constexpr (kNeedsLo<E>) mma(gacc[db], kf, sl);
                  }
                }
              }
            }
          };
          if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
            body(std::true_type{});
          else
            body(std::false_type{});
        }
        if (next) {
          if (NB == 1) __syncthreads();
          store(i + 1 < n ? pass : 1, nb);
        }
        __syncthreads();
      }
    }
    if (pass == 0) {
      num += __shfl_xor(num, 32);
      den += __shfl_xor(den, 32);
      dlt = den > 0.0f ? num / den : 0.0f;
      if (valid && h == 0) delta_out[(size_t)bh * N + iq] = dlt;
    }
  }
  // This workgroup's four mask rows, transposed ([kt][32-query row], one
  // 4-byte word per key tile), for the dK/dV kernel's lists.
  {
    const int np = (P.n_q32 + 3) & ~3;
    for (int kt = threadIdx.x; kt < P.n_kt; kt += kThreads) {
      uint32_t word = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww)
        if (active(ww, kt)) word |= 1u << (8 * ww);
      *reinterpret_cast<uint32_t*>(maskT + ((size_t)bh * P.n_kt + kt) * np + qtile * kWaves) = word;
    }
  }
  if (!valid) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * h;
      const size_t off = hoff + (size_t)iq * D + d0;
      const f32x4 o =
          f32x4{gacc[db][4 * g], gacc[db][4 * g + 1], gacc[db][4 * g + 2], gacc[db][4 * g + 3]} * P.inv_sqrt_d;
      if (P.out_bf16) {
        const bf16x4 ob = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(dq) + off) = ob;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dq) + off) = o;
      }
    }
}

// -------------------------------------------------------- k_bwd_dkdv ---
// Per workgroup (128 keys, 32 per wave): dV = P^T dO and dK = dS^T Q / sqrt(d)
// over the active 32-query blocks of the two mask columns it covers.  Scores
// are computed as S = Q K^T here (lane = key), so P and dS feed the A operand;
// the B operand runs down the columns of the staged Q / dO tiles (bf16:
// transposed LDS reads; fp32: staged Q^T / dO^T copies).
// Pipeline depth of the dK/dV query blocks.  The loop takes any depth with
// the LDS copy engine (bf16, d = 128), but the compiler waits for every copy
// in flight before a transposed LDS read, so blocks beyond the next one only
// cost LDS; one wave per SIMD without spills measured slower as well.
template <typename E, int D>
constexpr int kv_stages() { return 2; }
template <typename E, int D>
constexpr int kv_step_bytes() {
  return 2 * kBQ * row_stride<E, D>() + 2 * (sizeof(E) == 2 ? 0 : D * (kBQ * (int)sizeof(E) + 16)) + 2 * kBQ * 4;
}

template <typename E, int D, int AK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 2 : 1, 2))) void k_bwd_dkdv(
    const E* __restrict__ Q, const E* __restrict__ K, const E* __restrict__ V,
    const E* __restrict__ dO, const E* __restrict__ Qt, const E* __restrict__ dOt,
    const float* __restrict__ tau_in, const float* __restrict__ delta_in,
    const uint8_t* __restrict__ maskT, Params P, void* __restrict__ dk, void* __restrict__ dv) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool kTr = sizeof(E) == 2;
  constexpr bool kDirect = kTr && D == 128;          // LDS copy engine for every staged array
  constexpr int NS = kv_stages<E, D>();
  constexpr int KS = row_stride<E, D>();
  constexpr int TS = kBQ * (int)sizeof(E) + 16;
  constexpr int TT = kTr ? 0 : D * TS;               // bytes of one staged transposed tile
  constexpr int STEP = kv_step_bytes<E, D>();        // one pipeline buffer
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = P.N;
  int bh, ktile;
  map_tile((N + 127) / 128, P.BH, false, bh, ktile);
  const int kw0 = ktile * 128 + 32 * w;
  const int jk = kw0 + c32;
  const bool kvalid = jk < N;
  const bool wave_keys = kw0 < N;
  const size_t hoff = (size_t)bh * N * D;
  const E* Qth = kTr ? nullptr : Qt + (size_t)bh * D * P.Np;
  const E* dOth = kTr ? nullptr : dOt + (size_t)bh * D * P.Np;

  // buffer b: Q rows | dO rows | [Q^T cols | dO^T cols] | tau[32] | delta[32]
  short* list = reinterpret_cast<short*>(smem + NS * STEP);
  uint8_t* wbits = reinterpret_cast<uint8_t*>(list + kChunk);
  uint8_t* flags = wbits + kChunk;
  int* counter = reinterpret_cast<int*>(flags + kChunk);

  // bf16, d = 128: the workgroup's 128 K rows stay in LDS (each wave copies
  // its own 32) and the S products read them from there, which frees 32
  // VGPRs of K fragments; otherwise K fragments are held in registers.
  char* klds = smem + NS * STEP + 4 * kChunk + 16;
  Frag<E> kf[kDirect ? 1 : D / 16], vf[D / 16];
  if constexpr (kDirect) {
    RowTiles<E, D, 4 * kBQ> sk(K + hoff, N, w, lane);
    sk.fetch(klds, ktile * 128);
  } else {
    load_qfrags<E, D>(kf, K + hoff + (size_t)jk * D, kvalid, h);
  }
  load_qfrags<E, D>(vf, V + hoff + (size_t)jk * D, kvalid, h);

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }
  const int ktA = (ktile * 128) / kBK, ktB = ktA + 1;
  const int np = (P.n_q32 + 3) & ~3;
  // waves 0, 1 cover key tile A (64 keys), waves 2, 3 key tile B; the
  // transposed mask gives each key tile's query rows contiguously
  auto active = [&](int ww, int r) -> bool {
    const int kt = ww < 2 ? ktA : ktB;
    if (kt >= P.n_kt || (ktile * 128 + 32 * ww) >= N) return false;
    return maskT[((size_t)bh * P.n_kt + kt) * np + r] != 0;
  };

  RowTiles<E, D, kBQ> sq(Q + hoff, N, w, lane), so(dO + hoff, N, w, lane);
  ColStage<E, D, kBQ> sqt, sot;
  // per-query tau and delta of a block: copy engine (waves 0 and 1, 32 lanes
  // each; rows past N read as zeros and are masked by the row limits) or
  // registers of the first 32 threads
  __amdgpu_buffer_rsrc_t rs_td = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(w == 0 ? tau_in + (size_t)bh * N : delta_in + (size_t)bh * N), (short)0, N * 4,
      0x00020000);
  float sta = 0.0f, sde = 0.0f;
  auto load = [&](int r, int b) {
    const int qb0 = r * kBQ;
    char* p = smem + b * STEP;
    sq.fetch(p, qb0);
    so.fetch(p + kBQ * KS, qb0);
    if constexpr (kDirect) {
      if (w < 2 && lane < kBQ) {
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(
            (uint32_t)reinterpret_cast<uintptr_t>(p + 2 * kBQ * KS + 2 * TT + w * kBQ * 4));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs_td, reinterpret_cast<__attribute__((address_space(3))) void*>(d0), 4, lane * 4,
            __builtin_amdgcn_readfirstlane(qb0 * 4), 0, 0);
      }
    } else {
      if constexpr (!kTr) {
        sqt.load(Qth, P.Np, qb0);
        sot.load(dOth, P.Np, qb0);
      }
      if (threadIdx.x < kBQ) {
        const int qi = qb0 + threadIdx.x;
        sta = qi < N ? tau_in[(size_t)bh * N + qi] : INFINITY;
        sde = qi < N ? delta_in[(size_t)bh * N + qi] : 0.0f;
      }
    }
  };
  auto store = [&](int b) {
    if constexpr (!kDirect) {
      char* p = smem + b * STEP;
      sq.commit(p);
      so.commit(p + kBQ * KS);
      if constexpr (!kTr) {
        sqt.store(p + 2 * kBQ * KS, TS);
        sot.store(p + 2 * kBQ * KS + TT, TS);
      }
      if (threadIdx.x < kBQ) {
        float* f = reinterpret_cast<float*>(p + 2 * kBQ * KS + 2 * TT);
        f[threadIdx.x] = sta;
        f[kBQ + threadIdx.x] = sde;
      }
    }
  };
  // copy-engine loads one wave issues per block (Q and dO rows; the tau and
  // delta loads of waves 0 and 1 come on top, so waiting for this many keeps
  // on the safe side)
  constexpr int kPerBlock = 2 * kBQ / kWaves;

  for (int base = 0; base < P.n_q32; base += kChunk) {
    const int n = build_list(base, min(kChunk, P.n_q32 - base), active, list, wbits, flags, counter);
    if constexpr (kDirect) {
#pragma unroll
      for (int j = 0; j < NS - 1; ++j)
        if (j < n) load(base + list[j], j);
    } else {
      if (n > 0) {
        load(base + list[0], 0);
        store(0);
      }
      __syncthreads();
    }
    for (int i = 0; i < n; ++i) {
      const int r = base + list[i];
      const int qb0 = r * kBQ;
      int buf;
      if constexpr (kDirect) {
        // block i landed (blocks i+1 .. i+NS-2 may still be in flight), then
        // its slot's previous block is done everywhere and i+NS-1 takes it
        const int ahead = min(NS - 2, n - 1 - i);
        if (ahead >= 2) wait_vmcnt<2 * kPerBlock>();
        else if (ahead == 1) wait_vmcnt<kPerBlock>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (i + NS - 1 < n) load(base + list[i + NS - 1], (i + NS - 1) % NS);
        buf = i % NS;
      } else {
        if (i + 1 < n) load(base + list[i + 1], (i + 1) & 1);
        buf = i & 1;
      }
      if (wave_keys && ((wbits[i] >> w) & 1)) {
        const char* p = smem + buf * STEP;
        const char* qtl = p;
        const char* otl = p + kBQ * KS;
        const char* qttl = p + 2 * kBQ * KS;
        const char* ottl = qttl + TT;
        const float* taus = reinterpret_cast<const float*>(p + 2 * kBQ * KS + 2 * TT);
        const float* dels = taus + kBQ;
        // S = Q K^T and dP = dO V^T: rows = the 32 queries, column = this lane's key
        f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          Frag<E> a, b;
          ld8(a, reinterpret_cast<const E*>(qtl + c32 * KS) + 16 * c + 8 * h);
          if constexpr (kDirect) {
            Frag<E> kc;
            ld8(kc, reinterpret_cast<const E*>(klds + (32 * w + c32) * KS) + 16 * c + 8 * h);
            mma(sacc, a, kc);
          } else {
            mma(sacc, a, kf[c]);
          }
          ld8(b, reinterpret_cast<const E*>(otl + c32 * KS) + 16 * c + 8 * h);
          mma(pacc, b, vf[c]);
        }
        // query rows r (acc_row) are visible to this lane's key when
        // jk - qb0 <= r <= N - 1 - qb0 (causal) and the key exists
        auto softmax_like = [&](auto masked) {
          const int rlo = (P.causal ? jk - qb0 : INT_MIN / 2) - 4 * h;
          const int rhi = (kvalid ? N - 1 - qb0 : -1) - 4 * h;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int qr = acc_row(j, h);
            float sv = sacc[j];
            if constexpr (decltype(masked)::value) {
              const int r0 = 8 * (j >> 2) + (j & 3);
              if (r0 < rlo || r0 > rhi) sv = -INFINITY;
            }
            const float t = clamp01(fmaf(sv, P.scale, -taus[qr]));
            float pp, u;
            Ent<AK>::pu(t, P.beta, pp, u);
            sacc[j] = pp;
            pacc[j] = u * (pacc[j] - dels[qr]);
          }
        };
        if (qb0 + kBQ > N || (P.causal && kw0 + 31 > qb0) || kw0 + 32 > N)
          softmax_like(std::true_type{});
        else
          softmax_like(std::false_type{});
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag<E> pf, sf;
          from_acc(pf, sacc, 8 * s);
          from_acc(sf, pacc, 8 * s);
          const int qoff = 16 * s + 4 * h;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            Frag<E> ob, qb;
            if constexpr (kTr) {
              ld_col8(ob, otl, KS, qoff, 32 * db, lane);
              ld_col8(qb, qtl, KS, qoff, 32 * db, lane);
            } else {
              const E* orow = reinterpret_cast<const E*>(ottl + (32 * db + c32) * TS);
              const E* qrow = reinterpret_cast<const E*>(qttl + (32 * db + c32) * TS);
              ld4x2(ob, orow + qoff, orow + qoff + 8);
              ld4x2(qb, qrow + qoff, qrow + qoff + 8);
            }
            mma(dva[db], pf, ob);
            mma(dka[db], sf, qb);
          }
        }
      }
      if constexpr (!kDirect) {
        if (i + 1 < n) store((i + 1) & 1);
        __syncthreads();
      }
    }
    if constexpr (kDirect) __syncthreads();   // the next chunk's list and loads reuse the buffers
  }
  if (!wave_keys) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = kw0 + acc_row(j, h);
      if (key >= N) continue;
      const size_t off = hoff + (size_t)key * D + 32 * db + c32;
      const float vv = dva[db][j], kk = dka[db][j] * P.inv_sqrt_d;
      if (P.out_bf16) {
        reinterpret_cast<__bf16*>(dv)[off] = (__bf16)vv;
        reinterpret_cast<__bf16*>(dk)[off] = (__bf16)kk;
      } else {
        reinterpret_cast<float*>(dv)[off] = vv;
        reinterpret_cast<float*>(dk)[off] = kk;
      }
    }
}

// =============================================================== host ===

struct Shape {
  int B, H, N, d, esz, n_kt, n_q32, n_qt128, n_qt256, n_kt128, Np;
  int BH;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxN = 1 << 20;

int check_desc(const ea_desc* desc, Shape* s) {
  if (!desc) return EA_ERR_NULL;
  if (desc->B < 1 || desc->H < 1 || desc->N < 0 || (desc->d != 64 && desc->d != 128))
    return EA_ERR_SHAPE;
  if (desc->N > kMaxN || (long long)desc->B * desc->H > (1 << 20)) return EA_ERR_SHAPE;
  if ((desc->in_dtype != EA_F32 && desc->in_dtype != EA_BF16) ||
      (desc->out_dtype != EA_F32 && desc->out_dtype != EA_BF16))
    return EA_ERR_DTYPE;
  if (desc->tau_mode < EA_TAU_HIST_HALLEY || desc->tau_mode > EA_TAU_BISECT) return EA_ERR_UNSUPPORTED;
  if (desc->max_iters < 0 || desc->max_iters > 250) return EA_ERR_UNSUPPORTED;
  if (!(desc->tol >= 0.0f) || !(desc->tol < 1.0f)) return EA_ERR_UNSUPPORTED;
  if (desc->flags & ~EA_FLAG_FORCE_DENSE) return EA_ERR_UNSUPPORTED;
  if (s) {
    s->B = desc->B;
    s->H = desc->H;
    s->N = desc->N;
    s->d = desc->d;
    s->esz = desc->in_dtype == EA_BF16 ? 2 : 4;
    s->n_kt = (desc->N + kBK - 1) / kBK;
    s->n_q32 = (desc->N + kBQ - 1) / kBQ;
    s->n_qt128 = (desc->N + kBQW - 1) / kBQW;
    s->n_qt256 = (desc->N + 255) / 256;
    s->n_kt128 = (desc->N + 127) / 128;
    s->Np = s->n_kt * kBK;
    s->BH = desc->B * desc->H;
  }
  return EA_OK;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_alpha(float alpha) {
  if (!(alpha > 1.0f) || !(alpha <= 2.0f)) return EA_ERR_ALPHA;
  return EA_OK;
}

// Transposed copies are needed only for fp32 inputs: bf16 tiles are read down
// their columns with ds_read_b64_tr_b16 instead.
size_t transposed_bytes(const Shape& s) {
  return s.esz == 4 ? align_up((size_t)s.BH * s.d * s.Np * s.esz, 256) : 0;
}
size_t row_bytes(const Shape& s) { return align_up((size_t)s.BH * s.N * sizeof(float), 256); }
// one half per (row, 64-key tile), rows padded to a multiple of 32 tiles
size_t tilemax_bytes(const Shape& s) {
  const size_t ktp = (size_t)tilemax_row(s.n_kt);
  return align_up((size_t)s.BH * s.N * ktp * sizeof(uint16_t), 256);
}

// the block mask transposed, [BH][n_kt][n_q32 rounded up to 4] bytes
size_t maskt_bytes(const Shape& s) {
  return align_up((size_t)s.BH * s.n_kt * (size_t)((s.n_q32 + 3) & ~3), 256);
}

size_t workspace_bytes(const Shape& s) {
  // forward: [V^T] | row maxima | tile maxima;
  // backward: [K^T | Q^T | dO^T] | delta | transposed mask
  const size_t fwd = transposed_bytes(s) + row_bytes(s) + tilemax_bytes(s);
  const size_t bwd = 3 * transposed_bytes(s) + row_bytes(s) + maskt_bytes(s);
  const size_t ws = bwd > fwd ? bwd : fwd;
  return ws > 256 ? ws : 256;
}

int alpha_kind(float alpha) {
  if (alpha == 1.5f) return AK15;
  if (alpha == 2.0f) return AK20;
  if (alpha == 1.25f) return AK125;
  return AKGEN;
}

Params make_params(const ea_desc* desc, const Shape& s, float alpha, int causal) {
  Params P;
  P.N = s.N;
  P.n_kt = s.n_kt;
  P.n_q32 = s.n_q32;
  P.causal = causal ? 1 : 0;
  P.Np = s.Np;
  P.BH = s.BH;
  P.alpha = alpha;
  P.beta = (float)(1.0 / ((double)alpha - 1.0));
  P.scale = (float)(((double)alpha - 1.0) / sqrt((double)s.d));
  P.inv_sqrt_d = (float)(1.0 / sqrt((double)s.d));
  P.mode = desc->tau_mode;
  P.max_iters = desc->max_iters > 0 ? desc->max_iters : (desc->tau_mode == EA_TAU_BISECT ? 40 : 12);
  P.flags = desc->flags;
  P.tol = desc->tol > 0.0f ? desc->tol : 1e-6f;
  P.out_bf16 = desc->out_dtype == EA_BF16 ? 1 : 0;
  P.pair_qt = 0;
  return P;
}

// Causal row-max sweep: query tile t costs t + 1 key-tile steps.  When the
// query tiles fill about two rounds of resident workgroups (two per compute
// unit), pairing t with n - 1 - t in one workgroup gives one round of equal
// workgroups and measured 5% faster than the heaviest-first order; at four
// or more rounds the heaviest-first order balances better by itself, and
// below two rounds the pairs would leave compute units idle.
bool pair_query_tiles(const Shape& s, int causal) {
  if (!causal) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return false;
  const long tiles = (long)s.n_qt256 * s.BH, slots = 2L * cus;
  return 2 * tiles > 3 * slots && 2 * tiles <= 5 * slots;
}

// Records the caller's timing events around one stage (no-op without events).
struct StageTimer {
  void* const* ev;
  hipStream_t st;
  void begin(int s) const {
    if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev[2 * s]), st);
  }
  void end(int s) const {
    if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev[2 * s + 1]), st);
  }
};

template <typename F>
int set_lds(F* fn, size_t bytes) {
  if (bytes > 160 * 1024) return EA_ERR_UNSUPPORTED;
  if (bytes > 64 * 1024) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes) != hipSuccess)
      return EA_ERR_LAUNCH;
  }
  return EA_OK;
}

template <typename E, int D, int AK>
int launch_fwd(const Shape& s, Params P, const void* q, const void* k, const void* v, void* out,
               float* tau, uint8_t* mask, uint8_t* iters, void* ws, hipStream_t st, StageTimer tm) {
  constexpr bool kTr = sizeof(E) == 2;
  const E* Q = static_cast<const E*>(q);
  const E* K = static_cast<const E*>(k);
  const E* V = static_cast<const E*>(v);
  if (s.N == 0) return EA_OK;
  char* w = static_cast<char*>(ws);
  E* Vt = reinterpret_cast<E*>(w);
  float* rowmax = reinterpret_cast<float*>(w + transposed_bytes(s));
  uint16_t* tilemax = reinterpret_cast<uint16_t*>(w + transposed_bytes(s) + row_bytes(s));
  int rc;

  tm.begin(EA_STAGE_FWD_PREP);
  if constexpr (!kTr)
    hipLaunchKernelGGL(k_transpose<E>, dim3(s.Np / 64, D / 64, s.BH), dim3(256), 0, st, V, Vt, s.N, D, s.Np);
  tm.end(EA_STAGE_FWD_PREP);

  constexpr int KS = row_stride<E, D>();
  if constexpr (sizeof(E) == 2) {
    const size_t rm_lds = (size_t)2 * kRowmaxTPS * DirectTile<D>::BYTES;
    auto krm = k_rowmax16<D>;
    if ((rc = set_lds(krm, rm_lds)) != EA_OK) return rc;
    tm.begin(EA_STAGE_ROWMAX);
    P.pair_qt = pair_query_tiles(s, P.causal) ? 1 : 0;
    const int units = P.pair_qt ? (s.n_qt256 + 1) / 2 : s.n_qt256;
    hipLaunchKernelGGL(krm, dim3(units * s.BH), dim3(kThreads), rm_lds, st, Q, K, P, rowmax, tilemax);
    tm.end(EA_STAGE_ROWMAX);
  } else {
    const size_t rm_lds = (size_t)2 * kBK * KS;
    auto krm = k_rowmax<E, D>;
    if ((rc = set_lds(krm, rm_lds)) != EA_OK) return rc;
    tm.begin(EA_STAGE_ROWMAX);
    hipLaunchKernelGGL(krm, dim3(s.n_qt256 * s.BH), dim3(kThreads), rm_lds, st, Q, K, P, rowmax, tilemax);
    tm.end(EA_STAGE_ROWMAX);
  }

  constexpr int BINS = 16;
  const size_t tau_lds = (size_t)2 * kBK * KS + (size_t)tau_region_bytes<E, D>(BINS) + 4 * kChunk +
                         (size_t)2 * kWaves * ((s.n_kt + 31) / 32) * 4 + 64;
  auto ktau = k_tau<E, D, AK, BINS>;
  if ((rc = set_lds(ktau, tau_lds)) != EA_OK) return rc;
  const dim3 g(s.n_qt128 * s.BH);
  tm.begin(EA_STAGE_TAU);   // bf16: tau, block mask and P V in one kernel
  hipLaunchKernelGGL(ktau, g, dim3(kThreads), tau_lds, st, Q, K, V, rowmax, tilemax, P, tau, mask, iters, out);
  tm.end(EA_STAGE_TAU);

  tm.begin(EA_STAGE_PV);   // empty for bf16 (fused above)
  if constexpr (!kTr) {
    constexpr int VT = D * (kBK * (int)sizeof(E) + 16);
    const size_t pv_lds = (size_t)2 * kBK * KS + (size_t)2 * VT + 4 * kChunk + 16;
    auto kpv = k_pv<E, D, AK>;
    if ((rc = set_lds(kpv, pv_lds)) != EA_OK) return rc;
    hipLaunchKernelGGL(kpv, g, dim3(kThreads), pv_lds, st, Q, K, Vt, tau, mask, P, out);
  }
  tm.end(EA_STAGE_PV);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

template <typename E, int D, int AK>
int launch_bwd(const Shape& s, Params P, const void* q, const void* k, const void* v,
               const void* dout, const float* tau, const uint8_t* mask, void* dq, void* dk, void* dv,
               void* ws, hipStream_t st, StageTimer tm) {
  constexpr bool kTr = sizeof(E) == 2;
  const E* Q = static_cast<const E*>(q);
  const E* K = static_cast<const E*>(k);
  const E* V = static_cast<const E*>(v);
  const E* dO = static_cast<const E*>(dout);
  if (s.N == 0) return EA_OK;
  char* w = static_cast<char*>(ws);
  const size_t tb = transposed_bytes(s);
  E* Kt = reinterpret_cast<E*>(w);
  E* Qt = reinterpret_cast<E*>(w + tb);
  E* dOt = reinterpret_cast<E*>(w + 2 * tb);
  float* delta = reinterpret_cast<float*>(w + 3 * tb);
  uint8_t* maskT = reinterpret_cast<uint8_t*>(w + 3 * tb + row_bytes(s));
  int rc;
  tm.begin(EA_STAGE_BWD_PREP);
  if constexpr (!kTr) {
    const dim3 tg(s.Np / 64, D / 64, s.BH);
    hipLaunchKernelGGL(k_transpose<E>, tg, dim3(256), 0, st, K, Kt, s.N, D, s.Np);
    hipLaunchKernelGGL(k_transpose<E>, tg, dim3(256), 0, st, Q, Qt, s.N, D, s.Np);
    hipLaunchKernelGGL(k_transpose<E>, tg, dim3(256), 0, st, dO, dOt, s.N, D, s.Np);
  }
  tm.end(EA_STAGE_BWD_PREP);

  constexpr int KS = row_stride<E, D>();
  constexpr int TT = kTr ? 0 : D * (kBK * (int)sizeof(E) + 16);
  constexpr int NB = (2 * (2 * kBK * KS + TT) + 4 * kChunk + 16) <= 160 * 1024 ? 2 : 1;
  const size_t dq_lds = (size_t)NB * (2 * kBK * KS + TT) + 4 * kChunk + 16;
  auto kdq = k_bwd_dq<E, D, AK, NB>;
  if ((rc = set_lds(kdq, dq_lds)) != EA_OK) return rc;
  tm.begin(EA_STAGE_DQ);
  hipLaunchKernelGGL(kdq, dim3(s.n_qt128 * s.BH), dim3(kThreads), dq_lds, st, Q, K, V, dO, Kt, tau, mask,
                     P, delta, maskT, dq);
  tm.end(EA_STAGE_DQ);

  const size_t kv_lds = (size_t)kv_stages<E, D>() * kv_step_bytes<E, D>() + 4 * kChunk + 16 +
                        (kTr && D == 128 ? (size_t)4 * kBQ * KS : 0);   // the K rows (bf16, d = 128)
  auto kkv = k_bwd_dkdv<E, D, AK>;
  if ((rc = set_lds(kkv, kv_lds)) != EA_OK) return rc;
  tm.begin(EA_STAGE_DKDV);
  hipLaunchKernelGGL(kkv, dim3(s.n_kt128 * s.BH), dim3(kThreads), kv_lds, st, Q, K, V, dO, Qt, dOt, tau,
                     delta, maskT, P, dk, dv);
  tm.end(EA_STAGE_DKDV);
  return hipGetLastError() == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

#define EA_DISPATCH(FN, ...)                                                          \
  do {                                                                                \
    const int ak = alpha_kind(alpha);                                                 \
    if (desc->in_dtype == EA_BF16) {                                                  \
      if (s.d == 64) {                                                                \
        switch (ak) {                                                                 \
          case AK15: return FN<__bf16, 64, AK15>(__VA_ARGS__);                        \
          case AK20: return FN<__bf16, 64, AK20>(__VA_ARGS__);                        \
          case AK125: return FN<__bf16, 64, AK125>(__VA_ARGS__);                      \
          default: return FN<__bf16, 64, AKGEN>(__VA_ARGS__);                         \
        }                                                                             \
      } else {                                                                        \
        switch (ak) {                                                                 \
          case AK15: return FN<__bf16, 128, AK15>(__VA_ARGS__);                       \
          case AK20: return FN<__bf16, 128, AK20>(__VA_ARGS__);                       \
          case AK125: return FN<__bf16, 128, AK125>(__VA_ARGS__);                     \
          default: return FN<__bf16, 128, AKGEN>(__VA_ARGS__);                        \
        }                                                                             \
      }                                                                               \
    } else {                                                                          \
      if (s.d == 64) {                                                                \
        switch (ak) {                                                                 \
          case AK15: return FN<float, 64, AK15>(__VA_ARGS__);                         \
          case AK20: return FN<float, 64, AK20>(__VA_ARGS__);                         \
          case AK125: return FN<float, 64, AK125>(__VA_ARGS__);                       \
          default: return FN<float, 64, AKGEN>(__VA_ARGS__);                          \
        }                                                                             \
      } else {                                                                        \
        switch (ak) {                                                                 \
          case AK15: return FN<float, 128, AK15>(__VA_ARGS__);                        \
          case AK20: return FN<float, 128, AK20>(__VA_ARGS__);                        \
          case AK125: return FN<float, 128, AK125>(__VA_ARGS__);                      \
          default: return FN<float, 128, AKGEN>(__VA_ARGS__);                         \
        }                                                                             \
      }                                                                               \
    }                                                                                 \
  } while (0)

}  // namespace

extern "C" {

size_t entmax_attn_workspace_bytes(const ea_desc* desc) {
  Shape s;
  if (check_desc(desc, &s) != EA_OK) return 0;
  return workspace_bytes(s);
}

int entmax_attn_mask_dims(const ea_desc* desc, int* n_qt, int* n_kt, int* bm, int* bn) {
  Shape s;
  int st = check_desc(desc, &s);
  if (st != EA_OK) return st;
  if (n_qt) *n_qt = s.n_q32;
  if (n_kt) *n_kt = s.n_kt;
  if (bm) *bm = kBQ;
  if (bn) *bn = kBK;
  return EA_OK;
}

int entmax_attn_fwd(const void* q, const void* k, const void* v, float alpha, int causal, void* out,
                    float* tau, uint8_t* block_mask, uint8_t* tau_iters, const ea_desc* desc, void* ws,
                    size_t ws_bytes, void* stream) {
  Shape s;
  int st = check_desc(desc, &s);
  if (st != EA_OK) return st;
  if ((st = check_alpha(alpha)) != EA_OK) return st;
  if (causal != 0 && causal != 1) return EA_ERR_UNSUPPORTED;
  if (s.N > 0) {
    if (!q || !k || !v || !out || !tau || !block_mask || !ws) return EA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(tau) ||
        misaligned(ws))
      return EA_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(s)) return EA_ERR_WORKSPACE;
  }
  Params P = make_params(desc, s, alpha, causal);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  EA_DISPATCH(launch_fwd, s, P, q, k, v, out, tau, block_mask, tau_iters, ws, hs,
              StageTimer{desc->events, hs});
}

int entmax_attn_bwd(const void* q, const void* k, const void* v, float alpha, int causal,
                    const void* dout, const float* tau, const uint8_t* block_mask, void* dq, void* dk,
                    void* dv, const ea_desc* desc, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int st = check_desc(desc, &s);
  if (st != EA_OK) return st;
  if ((st = check_alpha(alpha)) != EA_OK) return st;
  if (causal != 0 && causal != 1) return EA_ERR_UNSUPPORTED;
  if (s.N > 0) {
    if (!q || !k || !v || !dout || !tau || !block_mask || !dq || !dk || !dv || !ws) return EA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(dout) || misaligned(tau) ||
        misaligned(dq) || misaligned(dk) || misaligned(dv) || misaligned(ws))
      return EA_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(s)) return EA_ERR_WORKSPACE;
  }
  Params P = make_params(desc, s, alpha, causal);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  EA_DISPATCH(launch_bwd, s, P, q, k, v, dout, tau, block_mask, dq, dk, dv, ws, hs,
              StageTimer{desc->events, hs});
}

const char* entmax_attn_strerror(int status) {
  switch (status) {
    case EA_OK: return "success";
    case EA_ERR_NULL: return "a required pointer is NULL";
    case EA_ERR_SHAPE: return "invalid shape (B, H >= 1, N >= 0, d in {64, 128})";
    case EA_ERR_DTYPE: return "invalid element type";
    case EA_ERR_ALPHA: return "alpha must satisfy 1 < alpha <= 2";
    case EA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case EA_ERR_WORKSPACE: return "workspace too small";
    case EA_ERR_LAUNCH: return "kernel launch failed";
    case EA_ERR_UNSUPPORTED: return "unsupported option (tau_mode, max_iters, tol, flags or causal)";
    default: return "unknown status";
  }
}

}  // extern "C"
