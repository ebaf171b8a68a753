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
//    takes only row maxima and, per 32-query block and 64-key tile, a one-byte
//    code bounding the block's largest score in that tile below the rows'
//    maxima.  Tiles whose code rules out any score above a row's lower
//    bracket end can never hold a nonzero probability, so the histogram and
//    Halley sweeps visit candidate tiles only.
//  * The histogram holds integer moments (count, sum y, sum y^2 of
//    y = x - lo in fixed point, Y = floor(y (2^S - 1)) with S chosen from N)
//    updated with LDS integer atomics, so it is deterministic and, for alpha
//    in {1.5, 2}, gives f exactly at bin edges.  There it is built in two
//    passes: the strong tiles first, whose partial moments bound tau from
//    below and prune the rest, then the remaining candidates of that bound.
//  * The bf16 tau kernel is persistent: one workgroup per resident slot
//    takes heavy-first query tiles from per-XCD work queues, which keeps the
//    slots busy where the hardware dispatcher would hold workgroups back.
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

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

#include "entmax_attn.h"

namespace {

constexpr int kWave = 64;
constexpr int kBQ = 32;               // queries per wave = mask row granularity
constexpr int kWaves = 4;
constexpr int kBQW = kBQ * kWaves;    // queries per workgroup (forward, dQ)
constexpr int kBK = 64;               // keys per tile = mask column granularity
constexpr int kThreads = kWave * kWaves;

// Block mask byte of a (32-query, 64-key) tile: bit 0 = the tile holds a
// nonzero probability; bits 1 and 2 = keys 0-31 / 32-63 of the tile do (the
// 32x32 micro-tiles that P V and the backward skip on their own).
__host__ __device__ constexpr uint32_t half_bits(uint32_t m) { return m ? ((m >> 1) & 3u) : 0u; }

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
  int hshift;             // histogram fixed point: Y = floor(y (2^hshift - 1))
  // Caller tensors: rows per head (ld >= N) and block-mask strides.  They
  // differ from N and the mask shape only for one batch of a
  // variable-length call, which runs as its own problem of length N inside
  // the caller's [B, H, ld, d] tensors; workspace arrays always use N.
  int ld, mrs;
  long long mhs;
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

// Operand fragments whose 8 contraction elements run down one column of a
// row-major bf16 LDS tile: rows r0 + {0,1,2,3} and r0 + 8 + {0,1,2,3} (the
// permuted key order of the score accumulators), column 32 j + (lane & 31)
// for fragment j < NF.  ds_read_b64_tr_b16 gives lane i of each 16-lane group
// element i % 4 of the 8-byte chunks addressed by lanes 4k + i / 4 of that
// group (k = 0..3), so lane r of a group addresses row r0 + r / 4, column
// 32 j + 16 * half + 4 * (r % 4).
// Before a transposed read of its own the compiler waits for every copy in
// flight to LDS (it cannot tell the tile read from the tiles those copies
// fill), which exposes the next tile's copy wherever a tile's copy is still
// in flight at its first transposed read.  kAsm issues all the reads from one
// block of inline assembly instead, which is not tied to the copies and waits
// for its own reads before it ends (so no destination register is handed
// back before its data has arrived); the price is that the block's reads
// cannot overlap the work around it.
template <int NF, bool kAsm>
__device__ __forceinline__ void ld_col8_row(Frag<__bf16> (&f)[NF], const char* tile, int rs, int r0,
                                            int lane) {
  static_assert(NF == 2 || NF == 4, "fragments per row");
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const int g = lane & 15;
  if constexpr (!kAsm) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const char* p = tile + (r0 + (g >> 2)) * rs + (32 * j + 16 * ((lane >> 4) & 1) + 4 * (g & 3)) * 2;
      const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
      const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 8 * rs));
      f[j].v = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    return;
  }
  const uint32_t a0 = (uint32_t)reinterpret_cast<uintptr_t>(tile) + (uint32_t)((r0 + (g >> 2)) * rs) +
                      (uint32_t)((16 * ((lane >> 4) & 1) + 4 * (g & 3)) * 2);
  const uint32_t a1 = a0 + (uint32_t)(8 * rs);
  u32x2 x[2 * NF];
  if constexpr (NF == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:64\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:128\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
          "=&v"(x[7])
        : "v"(a0), "v"(a1)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(a0), "v"(a1)
        : "memory");
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const bf16x4 lo = __builtin_bit_cast(bf16x4, x[2 * j]), hi = __builtin_bit_cast(bf16x4, x[2 * j + 1]);
    f[j].v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}
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

// fp32 inputs: scores q.k are summed 16 contraction elements at a time from
// zero, and the chunk sums in double.  Summing all d products in one fp32
// accumulator rounds at the magnitude of the largest partial sum; where scores
// are large and tau lies just below them (clustered keys, |x| near 17 at
// d = 128) that rounding alone moves t = x - tau, and through it dK, by about
// the fp32 tolerance.
__device__ __forceinline__ void mma_chunk64(double (&s)[16], const Frag<float>& a, const Frag<float>& b) {
  f32x16 t = f32x16{};
  mma(t, a, b);
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] += (double)t[j];
}
__device__ __forceinline__ void round_acc(f32x16& acc, const double (&s)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = (float)s[j];
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
  if constexpr (sizeof(E) == 4) {
    // fp32: one 32-key half at a time, chunk sums in double
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      double sd[16] = {};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        Frag<E> a;
        ld8(a, reinterpret_cast<const E*>(klds + (32 * kb + c32) * ks) + 16 * c + 8 * h);
        mma_chunk64(sd, a, qf[c]);
      }
      round_acc(acc[kb], sd);
    }
    return;
  }
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
  [[maybe_unused]] double sd[sizeof(E) == 4 ? 16 : 1] = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    Frag<E> a, b;
    ld8(a, reinterpret_cast<const E*>(kl + roff) + 16 * st + 8 * h);
    ld8(b, reinterpret_cast<const E*>(vl + roff) + 16 * st + 8 * h);
    if constexpr (sizeof(E) == 4) mma_chunk64(sd, a, qf[st]);
    else mma(sa, a, qf[st]);
    mma(pa, b, of[st]);
  }
  if constexpr (sizeof(E) == 4) round_acc(sa, sd);
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

// Persistent workgroups: a kernel launched with one workgroup per resident
// slot takes its work units from a queue, in the order map_tile deals them
// (heavy first when causal), instead of leaving the order to the hardware
// dispatcher, which holds later workgroups back while earlier ones still run
// and leaves slots idle when unit lengths vary widely.  With B*H a multiple
// of 8 there is one queue per XCD, serving that XCD's heads; otherwise one.
// queue[] holds kQueues counters that the preceding kernel in the same call
// zeroes.  Every thread gets the unit; false once the queue is empty.
constexpr int kQueues = 8;
constexpr int kQueueBytes = 256;
__device__ __forceinline__ bool next_unit(int* queue, int* s_unit, int n_tiles, int BH, bool heavy_first,
                                          int& bh, int& tile) {
  const bool per_xcd = (BH & 7) == 0;
  const int xq = per_xcd ? (int)(blockIdx.x & 7) : 0;
  const int n_units = per_xcd ? n_tiles * (BH >> 3) : n_tiles * BH;
  if (threadIdx.x == 0) *s_unit = atomicAdd(queue + xq, 1);
  __syncthreads();
  const int u = __builtin_amdgcn_readfirstlane(*s_unit);   // uniform: the unit's values stay scalar
  if (u >= n_units) return false;
  int rank;
  if (per_xcd) {
    const int hx = BH >> 3;
    bh = xq * hx + u % hx;
    rank = u / hx;
  } else {
    bh = u % BH;
    rank = u / BH;
  }
  tile = heavy_first ? n_tiles - 1 - rank : rank;
  return true;
}
__device__ __forceinline__ void reset_queues(int* queue) {
  if (queue && blockIdx.x == 0 && threadIdx.x < kQueues) queue[threadIdx.x] = 0;
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
template <int D, int W = kWaves>
struct DirectTile {
  static constexpr int RB = D * 2;                 // row bytes
  static constexpr int CPR = RB / 16;              // chunks per row
  static constexpr int BYTES = kBK * RB;
  static constexpr int NI = BYTES / 1024 / W;      // instructions per wave (W waves share a tile)
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
  // load key/value rows row0 .. row0+63 into `tile` (the LDS offset is the
  // low 32 bits of the pointer)
  __device__ __forceinline__ void issue(char* tile, int row0, int w) const {
    const uint32_t d0 = (uint32_t)reinterpret_cast<uintptr_t>(tile);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(d0 + (uint32_t)((w * NI + i) * 1024)), 16,
          voff[i], row0 * RB, 0, 0);
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
// waves, BITS bits each at bit BITS * w) are not all zero into list[] /
// wbits[]; returns the count.  Every thread of the workgroup must call it.
// `flags` holds len bytes of scratch.
template <int BITS = 1, typename Pred>
__device__ __forceinline__ int build_list(int base, int len, Pred pred, short* list, uint8_t* wbits,
                                          uint8_t* flags, int* counter) {
  // (the thread index through an empty asm statement: in a persistent
  // kernel's unit loop nothing derived from it is kept live across units)
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  for (int i = tid; i < len; i += kThreads) {
    uint32_t b = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) b |= ((uint32_t)pred(ww, base + i) & ((1u << BITS) - 1u)) << (BITS * ww);
    flags[i] = (uint8_t)b;
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
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

// Block codes.  For each 32-query block and 64-key tile the row-max sweep
// keeps one byte c = floor(-128 r), clamped to 0..255, of
//   r = max over the block's rows i of (M_it - m_i(t))   (x-domain),
// where M_it is row i's largest score in tile t and m_i(t) the row's running
// maximum once tile t has been seen.  Since m_i(t) <= max_j x_ij, -c/128 >= r
// bounds M_it - max_j x_ij from above for every row of the block: a tile whose
// code gives -c/128 <= min_i (lo_i - max_j x_ij) cannot hold an x_ij above the
// lower bracket end lo_i of any of the block's rows, so it holds no nonzero
// probability.  The sweep visits the diagonal (masked) key tiles of a query
// tile first, where the running maximum of a causal row usually settles, then
// the rest in order.  One byte per mask entry: the workspace grows like the
// block mask, not like the score matrix.  Rows are padded to 64 tiles.
__host__ __device__ constexpr int blk_row(int n_kt) { return (n_kt + 63) & ~63; }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// maximum over each 32-lane half of the wave (every lane of the half gets it)
__device__ __forceinline__ float half_max32(float v) {
  v = fmax_nan(v, dpp_f<0xB1>(v));     // quad_perm [1,0,3,2]
  v = fmax_nan(v, dpp_f<0x4E>(v));     // quad_perm [2,3,0,1]
  v = fmax_nan(v, dpp_f<0x141>(v));    // row_half_mirror
  v = fmax_nan(v, dpp_f<0x140>(v));    // row_mirror
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float half_min32(float v) { return -half_max32(-v); }

// code of a block's relative maximum r <= 0 (-inf: no visible entry -> 255)
__device__ __forceinline__ uint32_t blk_code(float r) {
  return (uint32_t)fminf(floorf(fmaxf(-128.0f * r, 0.0f)), 255.0f);
}

// Collects one lane's block codes for 32 consecutive tiles: lane l keeps tile
// (32 s + (l & 31)) of the block (l >> 5 in the 16x16 sweep, the lane half in
// the 32x32 one) and a segment of 32 bytes is stored at once.  The diagonal
// tiles [kt_full, kt_end) of a query tile lie in one segment (kt_full is a
// multiple of 4, at most 4 of them); their codes wait in `vd` until the
// in-order walk reaches that segment (or are stored at the end).
struct BlkCodes {
  uint8_t* row;      // this lane's block row, null when the block is past N
  int lane32, segd;
  uint32_t v, vd;
  bool diag;
  __device__ __forceinline__ BlkCodes(uint8_t* r, int lane, int kt_full, int kt_end)
      : row(r), lane32(lane & 31), segd(kt_full >> 5), v(255u), vd(255u), diag(kt_end > kt_full) {}
  __device__ __forceinline__ void put_diag(int kt, float r) {
    if ((kt & 31) == lane32) vd = blk_code(r);
  }
  // in-order tile kt < kt_full (r: the block's value; skipped tiles pass -inf)
  __device__ __forceinline__ void put(int kt, float r, int kt_full) {
    if ((kt & 31) == 0) v = ((kt >> 5) == segd) ? vd : 255u;
    if ((kt & 31) == lane32) v = blk_code(r);
    if ((kt & 31) == 31 || kt == kt_full - 1) store(kt & ~31, v);
  }
  __device__ __forceinline__ void store(int kt0, uint32_t val) const {
    if (row) row[kt0 + lane32] = (uint8_t)val;
  }
  // after the walk: the diagonal segment, if the in-order walk never reached it
  __device__ __forceinline__ void finish(int kt_full) const {
    if (diag && (kt_full == 0 || ((kt_full - 1) >> 5) != segd)) store(segd << 5, vd);
  }
};

// ---------------------------------------------------------- k_rowmax ---
// The one full score sweep: per-row maxima of x = (alpha-1) q.k / sqrt(d)
// and the block codes (above) of every 32-query block and 64-key tile.  Each
// wave owns 64 queries (two B-operand blocks share every K fragment read from
// LDS); the workgroup (256 queries) streams K tiles double-buffered through
// registers, the diagonal tiles first.  This 32x32 form serves fp32 inputs;
// bf16 runs k_rowmax16.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_rowmax(const E* __restrict__ Q, const E* __restrict__ K,
                                                     Params P, float* __restrict__ rowmax,
                                                     uint8_t* __restrict__ blkc, int* __restrict__ queue) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int KS = row_stride<E, D>();
  reset_queues(queue);   // for k_tau, which runs next
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = P.N;
  const int n_qt = (N + 255) / 256;
  int bh, qtile;
  map_tile(n_qt, P.BH, P.causal, bh, qtile);
  const int q0 = qtile * 256;
  const int wq0 = q0 + 64 * w;
  const E* Qh = Q + (size_t)bh * P.ld * D;
  const E* Kh = K + (size_t)bh * P.ld * D;

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
  // lie inside [0, N): they need no masking.  Only the diagonal / tail tiles
  // [kt_full, kt_end) do; they are swept first.
  const int kt_full = min(P.causal ? q0 / kBK : P.n_kt, N / kBK);
  const int n_steps = kt_end;
  auto tile_at = [&](int s) { return s < kt_end - kt_full ? kt_full + s : s - (kt_end - kt_full); };

  float mr[2] = {-INFINITY, -INFINITY};    // running row maxima (raw q.k)
  RowStage<E, D, kBK> st;
  if (n_steps > 0) {
    st.load(Kh, tile_at(0) * kBK, N);
    st.store(smem, KS);
  }
  __syncthreads();

  // lane half h keeps the codes of query block h (rows wq0 + 32 h ...)
  const int my_blk = (wq0 >> 5) + h;
  BlkCodes bc(32 * my_blk < N ? blkc + ((size_t)bh * P.n_q32 + my_blk) * blk_row(P.n_kt) : nullptr, lane,
              kt_full, kt_end);
  // one tile: scores for both query blocks, optional masking, maxima; returns
  // the value of this lane's block for the block codes
  auto tile = [&](int s, int kt, auto masked) -> float {
    const char* kl = smem + (s & 1) * kBK * KS;
    f32x16 acc[2][2];
    if constexpr (sizeof(E) == 4) {
      // fp32: one (query block, key half) at a time, chunk sums in double
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          double sd[16] = {};
#pragma unroll
          for (int c = 0; c < D / 16; ++c) {
            Frag<E> a;
            ld8(a, reinterpret_cast<const E*>(kl + (32 * kb + c32) * KS) + 16 * c + 8 * h);
            mma_chunk64(sd, a, qf[qb][c]);
          }
          round_acc(acc[qb][kb], sd);
        }
    } else {
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
    }
    float rel[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (decltype(masked)::value) mask_rows_above(acc[qb], row_limit(kt * kBK, iq[qb], N, P.causal, h));
      // NaN-propagating maximum: v_maximum3_f32 with no canonicalising of the
      // MFMA results that fmaxf would need
      float tm = fmax_nan(acc[qb][0][0], acc[qb][1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) tm = fmax_nan(tm, fmax_nan(acc[qb][0][i], acc[qb][1][i]));
      // the row's maximum over the tile (lanes l and l^32 hold its two halves)
      tm = half_swap_max(tm);
      mr[qb] = fmaxf(mr[qb], tm);
      rel[qb] = tm == -INFINITY ? -INFINITY : (tm - mr[qb]) * P.scale;
    }
    return half_max32(h ? rel[1] : rel[0]);
  };

  for (int s = 0; s < n_steps; ++s) {
    const int kt = tile_at(s);
    if (s + 1 < n_steps) st.load(Kh, tile_at(s + 1) * kBK, N);
    if (kt >= kt_full) {
      const float r = kt < kt_end_w ? tile(s, kt, std::true_type{}) : -INFINITY;
      bc.put_diag(kt, r);
    } else {
      bc.put(kt, tile(s, kt, std::false_type{}), kt_full);
    }
    if (s + 1 < n_steps) st.store(smem + ((s + 1) & 1) * kBK * KS, KS);
    __syncthreads();
  }
  bc.finish(kt_full);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    if (iq[qb] < N && h == 0) rowmax[(size_t)bh * N + iq[qb]] = mr[qb] * P.scale;
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
constexpr int kRowmaxWaves = kWaves;           // waves per workgroup, 64 queries each
constexpr int kRowmaxQ = 64 * kRowmaxWaves;     // queries per workgroup
template <int D>
__global__ __launch_bounds__(64 * kRowmaxWaves) void k_rowmax16(const __bf16* __restrict__ Q,
                                                                const __bf16* __restrict__ K, Params P,
                                                                float* __restrict__ rowmax,
                                                                uint8_t* __restrict__ blkc,
                                                                int* __restrict__ queue) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using DT = DirectTile<D, kRowmaxWaves>;
  reset_queues(queue);   // for k_tau, which runs next
  constexpr int TPS = kRowmaxTPS;
  constexpr int KST = D / 32;      // contraction steps of 32
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int N = P.N;
  const int n_qt = (N + kRowmaxQ - 1) / kRowmaxQ;
  // Causal query tile t holds (kRowmaxQ / 64) (t + 1) key tiles of work.  With pair_qt a
  // workgroup takes the pair (n_qt - 1 - t, t), so that every workgroup
  // sweeps the same number of tiles (the middle tile of an odd count runs
  // alone); otherwise one tile per workgroup, heaviest first.
  int bh, unit;
  map_tile(P.pair_qt ? (n_qt + 1) / 2 : n_qt, P.BH, P.causal && !P.pair_qt, bh, unit);
  const __bf16* Qh = Q + (size_t)bh * P.ld * D;
  const __bf16* Kh = K + (size_t)bh * P.ld * D;
  const DT dt(Kh, N, w, lane);
  const int ktc = blk_row(P.n_kt);

  auto sweep = [&](int qtile) {
    const int q0 = qtile * kRowmaxQ;
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
    const int kt_end = P.causal ? (min(N - 1, q0 + kRowmaxQ - 1) / kBK + 1) : P.n_kt;
    const int kt_end_w = wq0 >= N ? 0 : (P.causal ? (min(N - 1, wq0 + 63) / kBK + 1) : P.n_kt);
    const int kt_full = min(P.causal ? q0 / kBK : P.n_kt, N / kBK);
    const int n_diag = kt_end - kt_full;
    // the diagonal (masked) tiles first, then the rest in order
    auto tile_at = [&](int s) { return s < n_diag ? kt_full + s : s - n_diag; };

#pragma unroll
    for (int j = 0; j < TPS; ++j)
      if (j < kt_end) dt.issue(smem + j * DT::BYTES, tile_at(j) * kBK, w);

    // lane l keeps query wq0 + l's maxima; lanes 0-31 and 32-63 form the
    // wave's two query blocks
    const int my_blk = (wq0 >> 5) + (lane >> 5);
    BlkCodes bc(32 * my_blk < N ? blkc + ((size_t)bh * P.n_q32 + my_blk) * ktc : nullptr, lane, kt_full,
                kt_end);
    float m = -INFINITY;

    // scores of the tile staged at kl into acc[query block][key block]; the
    // four A fragments of step ks + 1 are read while step ks's sixteen MFMAs
    // run, so no MFMA waits for an LDS read
    auto mfma_tile = [&](f32x4 (&acc)[4][4], const char* kl) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[b][kb] = f32x4{0, 0, 0, 0};
      bf16x8 a[2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a[0][kb] = *reinterpret_cast<const bf16x8*>(DT::at(kl, 16 * kb + c16, g));
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) {
        if (ks + 1 < KST) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            a[(ks + 1) & 1][kb] = *reinterpret_cast<const bf16x8*>(DT::at(kl, 16 * kb + c16, 4 * (ks + 1) + g));
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[b][kb] = mma16(a[ks & 1][kb], qf[b][ks], acc[b][kb]);
      }
    };
    // the schedule of one mfma_tile (a hint to the scheduler, which otherwise
    // moves the reads back next to their MFMAs): its first step's reads, then
    // each fragment's four MFMAs followed by one read of the next step
    auto sched_tile = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS reads
#pragma unroll
      for (int i = 0; i < 4 * KST; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0); // MFMAs
        if (i < 4 * (KST - 1)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    // the tile's maximum for each query (after masking), the running row
    // maximum m and the block's value for the tile code
    auto epilogue = [&](f32x4 (&acc)[4][4], int kt, auto masked) -> float {
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
        float t = fmax_nan(acc[b][0][0], acc[b][0][1]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = (kb == 0 ? 2 : 0); i < 4; ++i) t = fmax_nan(t, acc[b][kb][i]);
        pm[b] = t;
      }
      // Reduce over the four lane groups and scatter: group g keeps query
      // block g.  permlane32 swap pairs groups (0,2) and (1,3) for blocks
      // (0,2) and (1,3); permlane16 swap then pairs (0,1) and (2,3).
      const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[0]), __float_as_uint(pm[2]), false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[1]), __float_as_uint(pm[3]), false, false);
      const float a0 = fmax_nan(__uint_as_float(s02[0]), __uint_as_float(s02[1]));
      const float a1 = fmax_nan(__uint_as_float(s13[0]), __uint_as_float(s13[1]));
      const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
      const float tm = fmax_nan(__uint_as_float(s01[0]), __uint_as_float(s01[1]));
      m = fmaxf(m, tm);
      return half_max32(tm == -INFINITY ? -INFINITY : (tm - m) * P.scale);
    };
    auto tile = [&](int s, int kt, auto masked) -> float {
      f32x4 acc[4][4];
      mfma_tile(acc, smem + (s % (2 * TPS)) * DT::BYTES);
      sched_tile();
      return epilogue(acc, kt, masked);
    };

    // Step over TPS tiles: wait for them (issued one step earlier; this also
    // retires the code stores), bare barrier (a full __syncthreads would add a
    // memory fence), issue the next step's tiles into the slots that the
    // previous step read, compute.
    for (int s0 = 0; s0 < kt_end; s0 += TPS) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int j = 0; j < TPS; ++j) {
        const int sn = s0 + TPS + j;
        if (sn < kt_end) dt.issue(smem + (sn % (2 * TPS)) * DT::BYTES, tile_at(sn) * kBK, w);
      }
#pragma unroll
      for (int j = 0; j < TPS; ++j) {
        const int s = s0 + j;
        if (s >= kt_end) break;
        const int kt = tile_at(s);
        if (kt >= kt_full) {
          const float r = kt < kt_end_w ? tile(s, kt, std::true_type{}) : -INFINITY;
          bc.put_diag(kt, r);
        } else {
          bc.put(kt, tile(s, kt, std::false_type{}), kt_full);
        }
      }
    }
    bc.finish(kt_full);
    const int iq = wq0 + lane;
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
  bool live[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float mx = acc[kb][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmax_nan(mx, acc[kb][j]);
    // the 32x32 micro-tile holds a nonzero probability for some query
    live[kb] = __ballot(fmaf(mx, P.scale, -tau) > 0.0f) != 0ull;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float t = clamp01(fmaf(acc[kb][j], P.scale, -tau));
      float p, u;
      Ent<AK>::pu(t, P.beta, p, u);
      acc[kb][j] = p;
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (!live[kb]) continue;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      Frag<E> pf;
      from_acc(pf, acc[kb], 8 * s);
      const int koff = 32 * kb + 16 * s + 4 * h;
      Frag<E> vf[D / 32];
      if constexpr (kTr) {
        ld_col8_row<D / 32, false>(vf, vl, VS, koff, lane);
      } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const E* vrow = reinterpret_cast<const E*>(vl + (32 * db + c32) * VS);
          ld4x2(vf[db], vrow + koff, vrow + koff + 8);
        }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) mma(oacc[db], vf[db], pf);
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

// ------------------------------------------------- histogram start ---
// A row's histogram over the bracket [lo, hi]: BINS uniform bins of
// y = x - lo, per bin two 64-bit words of integer moments of the fixed-point
// Y = floor(y (2^S - 1)) with S = hshift (count << 40 plus sum Y, and
// sum Y^2; see hist_add).  From it: tau's bin, a start value inside it and,
// for alpha in {1.5, 2} (where f is exact at the bin edges), the bracket
// narrowed to that bin.  The pages give only "a coarse histogram kept on
// chip" ("AdaSplash-2: The Transformer Revolution We Didn't See Coming",
// "Sparse Attention Makes Waves"); the bin count, the moments and the
// two-point start model are this library's.
//
// hist_add takes yc = y clamped to [0, 1] (entries at or below ylim >= 0 are
// dropped) and the LDS address of the row's histogram.  With 0 < yc <= 1 and ysc = 2^S - 1
// (S <= 24) the product rounds to at most 2^S - 1, so Y needs no clamp and
// Y^2 comes from the two 24-bit multiplies.  kAsm issues the two atomics by
// inline assembly: the compiler cannot tell the histogram from the tiles
// that copies in flight fill, and would wait for every copy before an atomic
// it emits itself.  (The histogram is disjoint from every copy destination;
// a wave's LDS operations execute in order, and the caller waits for them
// before the histogram is read.)
template <bool kAsm>
__device__ __forceinline__ void hist_add(uint32_t hrow, unsigned long long* hr, float yc, float bin_scale,
                                         float ysc, int bins, float ylim = 0.0f) {
  if (yc > ylim) {
    const unsigned Y = (unsigned)(yc * ysc);
    __builtin_assume(Y < (1u << 24));
    const int b = min((int)(yc * bin_scale), bins - 1);
    const unsigned long long w1 = (1ull << 40) + Y;
    const unsigned long long w2 = (unsigned long long)Y * (unsigned long long)Y;
    if constexpr (kAsm) {
      const uint32_t a = hrow + 16u * (uint32_t)b;
      asm volatile("ds_add_u64 %0, %1\n\tds_add_u64 %0, %2 offset:8" ::"v"(a), "v"(w1), "v"(w2) : "memory");
    } else {
      atomicAdd(&hr[2 * b], w1);
      atomicAdd(&hr[2 * b + 1], w2);
    }
  }
}
// wait for this wave's LDS operations, those issued by inline assembly included
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Bin edges as bracket ends: lo + e, widened by the float rounding of x and
// lo and by the fixed-point truncation of y (sign -1: a lower end, +1: upper).
__device__ __forceinline__ float hist_edge(float lo, double e, float xmax, int hshift, float sign) {
  const double yunit = 1.0 / (double)((1u << hshift) - 1u);
  const float margin = fmaxf(1.0f, fabsf(xmax)) * 5e-7f + 1e-6f + (float)(2.0 * yunit);
  return (float)((double)lo + e) + sign * margin;
}

// alpha in {1.5, 2}: the highest bin whose lower edge has f >= 0, with f
// taken from the moments of the bins above the edge (0 if no edge above the
// first qualifies).  Moments of only some of a row's scores give a value
// below f at every edge, so the edge found is a lower bound on tau even then.
template <int AK, int BINS>
__device__ __forceinline__ int hist_floor_bin(const unsigned long long* hr, float width, int hshift) {
  const double yunit = 1.0 / (double)((1u << hshift) - 1u), yunit2 = yunit * yunit;
  const double bw = (double)width / BINS;
  double C = 0, S1 = 0, S2 = 0;
#pragma unroll 1
  for (int b = BINS - 1; b > 0; --b) {
    const unsigned long long h1 = hr[2 * b], h2 = hr[2 * b + 1];
    C += (double)(h1 >> 40);
    S1 += (double)(h1 & ((1ull << 40) - 1ull)) * yunit;
    S2 += (double)h2 * yunit2;
    const double e = (double)b * bw;
    const double f = AK == AK15 ? S2 - 2.0 * e * S1 + e * e * C - 1.0 : S1 - e * C - 1.0;
    if (f >= 0.0) return b;
  }
  return 0;
}

template <int AK, int BINS>
__device__ __forceinline__ void hist_start(const unsigned long long* hr, float width, float xmax, int hshift,
                                        float beta, float& lo, float& hi, float& tau) {
  const double yunit = 1.0 / (double)((1u << hshift) - 1u), yunit2 = yunit * yunit;   // fixed-point units
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
        const float mu = (float)((double)(g1 & ((1ull << 40) - 1ull)) * yunit) / cc;
        const float sd = sqrtf(fmaxf((float)((double)g2 * yunit2) / cc - mu * mu, 0.0f));
        float da, db;
        const float va = model_pow<AK>(mu + sd - t, beta, da);
        const float vb = model_pow<AK>(mu - sd - t, beta, db);
        fv += 0.5f * cc * (va + vb);
        df -= 0.5f * cc * beta * (da + db);
      }
    }
    return fv;
  };
  for (int b = exact ? BINS - 1 : -1; b >= 0; --b) {   // the exact edge values
    const unsigned long long h1 = hr[2 * b], h2 = hr[2 * b + 1];
    const double cb = (double)(h1 >> 40);
    const double s1 = (double)(h1 & ((1ull << 40) - 1ull)) * yunit;
    const double s2 = (double)h2 * yunit2;
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
    const double s1b = (double)(g1 & ((1ull << 40) - 1ull)) * yunit;
    const double s2b = (double)g2 * yunit2;
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
    const float nlo = hist_edge(lo, eb, xmax, hshift, -1.0f);
    const float nhi = hist_edge(lo, eb1, xmax, hshift, 1.0f);
    if (nlo > lo) lo = nlo;
    if (nhi < hi) hi = nhi;
  }
  tau = fminf(fmaxf(t0x, lo), hi);
}

// ------------------------------------------------------------- k_tau ---
// Per workgroup (128 queries, 32 per wave): bracket from the row maxima,
// candidate key tiles from the block codes, histogram initialisation, Halley /
// bisection sweeps over candidate tiles, tau, iteration counts and the block
// mask.  Dynamic LDS: K double buffer | histogram [128][BINS*2+2] u64 |
// list i16[kChunk] | wave bits u8[kChunk] | flags u8[kChunk] |
// candidate bits u32[4][n_words] | counter | final mask bits u32[4][n_words] |
// bits of tiles above the lower bracket end u32[4][n_words] | bits of the two
// 32-key halves of active tiles u32[2][4][n_words].
constexpr int kChunk = 512;    // key tiles listed at once
// the histogram takes two passes when more lanes than this hold candidate
// tiles outside the strong ones (16 tiles a lane; below it the first pass
// would save little)
constexpr int kStrongMinWeak = 8;

// One refinement step of a row's tau from the sums of a sweep at tau
// (F0 = sum t^beta, F1 = sum t^(beta-1), F2 = sum t^(beta-2) or the support
// count), Halley-bisection or bisection ("Sparse Attention Makes Waves",
// accelerated alpha-entmax; AdaSplash paper abstract): stop when f is within
// tolerance or machine precision, else shrink the bracket with the sign of f
// and take the Halley (or Newton) step when it stays inside it, the midpoint
// otherwise.  A converged row keeps the tau it was evaluated at.
template <int AK>
__device__ __forceinline__ void tau_step(float F0, float F1, float F2, float beta_f, int mode, float tol,
                                         int max_iters, float& lo, float& hi, float& tau, bool& conv, int& iters) {
  if (conv) return;
  ++iters;
  const double beta = (double)beta_f;
  const double f = (double)F0 - 1.0;
  // tau is a float: one ulp of tau moves f by about |f'| ulp, so |f| below
  // that granularity (or a Halley step below two ulps) is machine precision.
  const double ulp = (double)FLT_EPSILON * fmax(1.0, fabs((double)tau));
  const double fp = -beta * (double)F1;
  const bool bisect = mode == EA_TAU_BISECT;
  if (fabs(f) <= (double)tol + (bisect ? 0.0 : 2.0 * fabs(fp) * ulp)) {
    conv = true;
    return;
  }
  if (f > 0.0) lo = tau; else hi = tau;
  const float wtol = bisect ? 1e-6f * fmaxf(1.0f, fabsf(tau)) : 4.0f * (float)ulp;
  if (hi - lo <= wtol || iters >= max_iters) {
    conv = true;
    return;
  }
  double next = 0.5 * ((double)lo + (double)hi);
  if (!bisect) {
    // Halley while |f f''| < f'^2; there the step lies between 2/3 and
    // 2 Newton steps, so a step of two ulps means |f| within three ulps
    // of |f'|.  Otherwise (for 1.5 < alpha < 2, f'' grows without bound
    // as a score nears tau from above) a Newton step.
    const double fpp = (AK == AK20) ? 0.0 : beta * (beta - 1.0) * (double)F2;
    const bool halley = fabs(f * fpp) < fp * fp;
    const double th = halley ? (double)tau - 2.0 * f * fp / (2.0 * fp * fp - f * fpp)
                             : (double)tau - f / fp;
    if (fabs(th - (double)tau) <= 2.0 * ulp) {
      conv = true;                        // converged: keep the evaluated tau
      return;
    }
    if (th > (double)lo && th < (double)hi) next = th;
  }
  float nt = (float)next;
  if (!(nt > lo && nt < hi)) nt = lo + 0.5f * (hi - lo);
  if (!(nt > lo && nt < hi)) conv = true;   // bracket exhausted in float
  else tau = nt;
}

template <typename E, int D>
constexpr int tau_region_bytes(int bins) {
  // histogram [128][2 bins + 2] u64; for bf16 also the V double buffer of the
  // P V epilogue, which reuses it
  return sizeof(E) == 2 && 2 * kBK * row_stride<E, D>() > kBQW * (2 * bins + 2) * 8
             ? 2 * kBK * row_stride<E, D>()
             : kBQW * (2 * bins + 2) * 8;
}

template <typename E, int D, int AK, int BINS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 2 : 1, 2))) void k_tau(const E* __restrict__ Q, const E* __restrict__ K,
                                                  const E* __restrict__ V,
                                                  const float* __restrict__ rowmax,
                                                  const uint8_t* __restrict__ blkc, Params Pk,
                                                  float* __restrict__ tau_out,
                                                  uint8_t* __restrict__ mask_out,
                                                  uint8_t* __restrict__ iters_out,
                                                  void* __restrict__ out, int* __restrict__ queue) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int KS = row_stride<E, D>();
  constexpr bool kFusePV = sizeof(E) == 2;   // bf16: P V runs here, after tau
  const int N = Pk.N;
  // one work unit: query tile qtile of head bh
  auto unit = [&](const int bh, const int qtile) {
    // The thread index passes through an empty asm statement, so that nothing
    // derived from it is hoisted out of the unit loop and kept live across it
    // (which would cost the registers of two waves per SIMD).
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
    // Likewise the parameters that feed double-precision set-up (the
    // histogram's fixed-point unit, the bracket, the Halley step): with
    // both, the kernel fits two waves per SIMD without spills.
    Params P = Pk;
    asm volatile("" : "+s"(P.alpha), "+s"(P.beta), "+s"(P.scale), "+s"(P.tol), "+s"(P.hshift));
    const int q0 = qtile * kBQW;
    const int wq0 = q0 + kBQ * w;
    const int iq = wq0 + c32;
    const bool valid = iq < N;
    const bool wave_rows = wq0 < N;
    const int r32 = qtile * kWaves + w;
    const E* Qh = Q + (size_t)bh * P.ld * D;
    const E* Kh = K + (size_t)bh * P.ld * D;
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
    uint32_t* lbits = mbits + kWaves * n_words;                         // [4][n_words] tiles above lo
    uint32_t* hbits = lbits + kWaves * n_words;                         // [2][4][n_words] live halves

    const int wq_last = min(N - 1, wq0 + kBQ - 1);
    const int kt_end_w = !wave_rows ? 0 : (P.causal ? wq_last / kBK + 1 : P.n_kt);
    const int kt_end = P.causal ? (min(N - 1, q0 + kBQW - 1) / kBK + 1) : P.n_kt;
    const bool wave_has_tail = wq0 + kBQ > N;
    // this wave's block codes; one 16-byte chunk per lane covers 1024 tiles
    const uint8_t* crow = blkc + ((size_t)bh * P.n_q32 + (size_t)min(r32, P.n_q32 - 1)) * blk_row(P.n_kt);
    u32x4 pre = u32x4{~0u, ~0u, ~0u, ~0u};
    if (16 * lane < kt_end_w) pre = *reinterpret_cast<const u32x4*>(crow + 16 * lane);

    Frag<E> qf[D / 16];
    load_qfrags<E, D>(qf, Qh + (size_t)iq * D, valid, h);

    // ---- provable bracket [lo, hi]:  f(max x - 1) >= 0 >= f(max x - n^(1-alpha))
    const float xmax = valid ? rowmax[(size_t)bh * N + iq] : 0.0f;
    float lo = 0.0f, hi = 0.0f, tau = 0.0f;
    if (valid) {
      const double dl = (double)xmax - 1.0;
      lo = (float)dl;
      if ((double)lo > dl) lo = nextafterf(lo, -INFINITY);
      // n^(1 - alpha) from the hardware log2 and exp2 (relative error a few
      // 1e-6 for n <= 2^20), made 2^-16 smaller: hi only has to bound tau
      // from above, and no double-precision pow stays live in the unit loop
      const float n = P.causal ? (float)(iq + 1) : (float)N;
      const float g = __builtin_amdgcn_exp2f((1.0f - P.alpha) * __builtin_amdgcn_logf(n)) * (1.0f - 0x1p-16f);
      const double dh = (double)xmax - (double)g;
      hi = (float)dh;
      if ((double)hi < dh) hi = nextafterf(hi, INFINITY);
      if (hi < lo) hi = lo;
    }
    bool conv = !valid;
    int iters = 0;

    // ---- candidate key tiles: bit kt of wave w is set when the block code of
    // tile kt admits a score above some row's lower bracket end (tau >= lo, so
    // no other tile can hold a nonzero probability for the wave).  The test
    // compares the code with the smallest lo_i - max_j x_ij of the wave's rows,
    // less a margin for the float rounding of both sides.  Words past the
    // wave's last visible tile are written as zeros up to the workgroup's end.
    // The first call (use_pre) also leaves each wave's strong tiles in mbits
    // for the two-pass histogram (below): its candidates with block code 0,
    // which hold the highest scores of some of its rows.  It returns the
    // number of the workgroup's lanes that hold other candidates.
    constexpr bool kStrongAK = AK == AK15 || AK == AK20;
    const bool strong_pass = kStrongAK && !dense && P.mode == EA_TAU_HIST_HALLEY;
    auto make_cand = [&](auto use_pre) -> int {
      __syncthreads();   // earlier readers of the bits are done
      // (the MFMA shapes of the row-max sweep and of this kernel round their
      // partial sums differently: 64 float epsilons of |x| covers that)
      float th = valid ? (lo - xmax) - 64.0f * FLT_EPSILON * (fmaxf(1.0f, fabsf(xmax)) + 2.0f) : INFINITY;
      th = half_min32(th);           // both lane halves hold the same 32 rows
      const float lim = -128.0f * th;   // candidate iff code < lim
      int weak = 0;
      for (int base = 0; base < kt_end; base += 64 * 16) {
        const int t0 = base + 16 * lane;
        u32x4 r = u32x4{~0u, ~0u, ~0u, ~0u};
        if (decltype(use_pre)::value && base == 0)
          r = pre;
        else if (t0 < kt_end_w)
          r = *reinterpret_cast<const u32x4*>(crow + t0);
        // (bits shifted in from the top: no mask constants to keep in registers)
        uint32_t bits = 0, sb = 0;
#pragma unroll
        for (int j = 15; j >= 0; --j) {
          const uint32_t c = (r[j >> 2] >> (8 * (j & 3))) & 0xFFu;
          const bool cj = (float)c < lim && t0 + j < kt_end_w;
          bits = (bits << 1) | (uint32_t)cj;
          sb = (sb << 1) | (uint32_t)(cj && c == 0u);
        }
        const int nv = min(max(kt_end_w - t0, 0), 16);
        if (dense) bits = nv >= 16 ? 0xFFFFu : ((1u << nv) - 1u);
        // lanes 2m and 2m+1 hold the two halves of word (base / 32) + m
        const uint32_t word = bits | (dpp_u<0xB1>(bits) << 16);
        const int wd = (base >> 5) + (lane >> 1);
        if (!(lane & 1) && wd < n_words) cbits[w * n_words + wd] = word;
        if constexpr (decltype(use_pre)::value) {
          if (strong_pass) {
            weak |= (bits & ~sb) != 0u;
            const uint32_t sword = sb | (dpp_u<0xB1>(sb) << 16);
            if (!(lane & 1) && wd < n_words) mbits[w * n_words + wd] = sword;
          }
        }
      }
      // (lanes that hold other candidates, per wave, beside build_list's counter)
      if (decltype(use_pre)::value && strong_pass) {
        const int nw = __popcll(__ballot(weak));
        if (lane == 0) counter[4 + w] = nw;
      }
      __syncthreads();
      if (decltype(use_pre)::value && strong_pass) return counter[4] + counter[5] + counter[6] + counter[7];
      return 0;
    };
    auto cand = [&](int ww, int kt) -> bool { return (cbits[ww * n_words + (kt >> 5)] >> (kt & 31)) & 1u; };
    const int weak_lanes = make_cand(std::true_type{});

    // ---- histogram initialisation (AdaSplash-2)
    if (P.mode == EA_TAU_HIST_HALLEY) {
      for (int e = tid; e < kBQW * HROW; e += kThreads) hist[e] = 0ull;
      unsigned long long* hr = hist + (size_t)(kBQ * w + c32) * HROW;
      // Bins split [lo, hi]; moments are kept in units of 1/(2^S - 1) of y = x - lo <= 1
      // with Y <= 2^S - 1: the count sits at bit 40, sum Y below it and sum Y^2
      // in a word of its own, so with at most N <= 2^(40-S) elements per bin
      // sum Y < 2^40 and sum Y^2 < 2^64.  S = 24 up to N = 65536, fewer bits
      // beyond (the host chooses S from N).
      const float width = valid ? fmaxf(hi - lo, 1e-30f) : 1.0f;
      const float bin_scale = (float)BINS / width;
      const float ysc = (float)((1u << P.hshift) - 1u);
      const uint32_t hrow = (uint32_t)reinterpret_cast<uintptr_t>(hr);
      const float lo0 = lo;   // the histogram's origin
      // Histogram passes: 0 takes every candidate tile.  For alpha in {1.5, 2}
      // there are two instead: pass 1 takes the strong tiles only (each wave's
      // candidates with block code 0, joined over the workgroup).  f of their
      // scores alone
      // lies below f, so their histogram's highest edge with f >= 0 is a lower
      // bound on tau; it prunes the candidates, and pass 2 adds the remaining
      // candidates of the raised bound.  Every score above that bound is then
      // in the histogram, so f at every edge above it, tau's bin, the start and
      // the narrowed bracket come out as from pass 0; only tiles that cannot
      // reach the bound are skipped.
      auto strong = [&](int kt) -> bool { return (lbits[kt >> 5] >> (kt & 31)) & 1u; };
      // two passes only when the workgroup holds enough other candidates to
      // skip some of them
      const bool two = strong_pass && weak_lanes > kStrongMinWeak;
      if (two) {
        // the union of the waves' strong tiles, in lbits (first written by the sweeps)
        for (int e = tid; e < n_words; e += kThreads)
          lbits[e] = mbits[e] | mbits[n_words + e] | mbits[2 * n_words + e] | mbits[3 * n_words + e];
        __syncthreads();
      }
      const int hp_first = two ? 1 : 0, hp_last = two ? 2 : 0;
#pragma clang loop unroll(disable)
      for (int hp = hp_first; hp <= hp_last; ++hp) {
        if (hp == 2) {
          wait_lds();
          if (valid) {
            const int b = hist_floor_bin<AK, BINS>(hr, width, P.hshift);
            if (b > 0) lo = fmaxf(lo, hist_edge(lo0, (double)b * ((double)width / BINS), xmax, P.hshift, -1.0f));
          }
          make_cand(std::false_type{});
          for (int e = lane; e < n_words; e += kWave) mbits[w * n_words + e] = 0u;
        }
        // Pass 2 also marks, per wave, the tiles where some row has a score
        // above its own raised bound (less a rounding margin), kept in mbits.
        // The block codes test a 32-row block against its loosest row; these
        // bits test every row against its own bound, and tau's bin only lies
        // higher, so they prune the first refinement sweep's candidates.  And
        // pass 2 bins only the scores above that bound: the edges below it
        // are never read (f at the bound is already >= 0), and every score in
        // a bin at or above it passes.
        const float gy = valid ? (lo - lo0) - 4.0f * FLT_EPSILON * (fmaxf(1.0f, fabsf(xmax)) + 2.0f) : 2.0f;
        const float ylim = hp == 2 ? fmaxf(gy, 0.0f) : 0.0f;   // (yc = 0 stays dropped)
        int bit_wd = -1;
        uint32_t r_word = 0u;
        auto flush_row_bits = [&]() {
          if (bit_wd >= 0 && lane == 0) mbits[w * n_words + bit_wd] = r_word;
          bit_wd = -1;
          r_word = 0u;
        };
        auto pred = [&](int ww, int kt) -> bool {
          return cand(ww, kt) && (hp == 0 || (hp == 1) == strong(kt));
        };
        for (int base = 0; base < kt_end; base += kChunk) {
          const int n = build_list(base, min(kChunk, kt_end - base), pred, list, wbits, flags, counter);
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
              float ymax = 0.0f;
              auto body = [&](auto masked) {
                f32x16 acc[2];
                tile_scores<E, D>(acc, kbuf + (i & 1) * kBK * KS, KS, qf, lane,
                                  row_limit(kt * kBK, iq, N, P.causal, h), masked);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                  for (int j = 0; j < 16; ++j) {
                    const float yc = clamp01(fmaf(acc[kb][j], P.scale, -lo0));
                    ymax = fmaxf(ymax, yc);
                    hist_add<true>(hrow, hr, yc, bin_scale, ysc, BINS, ylim);
                  }
              };
              if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
                body(std::true_type{});
              else
                body(std::false_type{});
              if (hp == 2) {
                // (the ballot runs on every lane: it must see every row)
                const bool above = __ballot(ymax > gy) != 0ull;
                const int wd = __builtin_amdgcn_readfirstlane(kt >> 5);
                if (wd != bit_wd) {
                  flush_row_bits();
                  bit_wd = wd;
                }
                if (above) r_word |= 1u << (kt & 31);
              }
            }
            if (i + 1 < n) st.commit(kbuf + ((i + 1) & 1) * kBK * KS);
            __syncthreads();
          }
          flush_row_bits();
        }
      }
      wait_lds();
      if (valid) {
        float lo_h = lo0;
        hist_start<AK, BINS>(hr, width, xmax, P.hshift, P.beta, lo_h, hi, tau);
        lo = fmaxf(lo, lo_h);
        tau = fminf(fmaxf(tau, lo), hi);
      }
      // the histogram narrowed lo to tau's bin: prune the candidates again
      if (AK == AK15 || AK == AK20) make_cand(std::false_type{});
      if (two) {
        // only tiles where some row passed its own raised bound, or strong ones
        for (int e = lane; e < n_words; e += kWave)
          cbits[w * n_words + e] &= mbits[w * n_words + e] | lbits[e];
        __syncthreads();
      }
    } else if (P.mode == EA_TAU_HALLEY_BISECT) {
      tau = lo;
    } else {
      tau = 0.5f * (lo + hi);
    }

    // ---- refinement sweeps (Halley-bisection or bisection) over candidate tiles
    // The final mask is kept as bits in LDS (the tile, and each 32-key half)
    // and written to block_mask after the sweeps; the P V epilogue reads it too.
    uint8_t* mrow = mask_out + (size_t)bh * P.mhs + (size_t)r32 * P.mrs;
    for (int e = lane; e < n_words; e += kWave) {
      const int nv = min(max(kt_end_w - 32 * e, 0), 32);
      const uint32_t vis = dense ? (nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u)) : 0u;
      mbits[w * n_words + e] = vis;
      hbits[w * n_words + e] = vis;
      hbits[(kWaves + w) * n_words + e] = vis;
    }
    const int max_iters = P.max_iters;
    // The candidate tiles only shrink between refinement sweeps.  When the
    // workgroup's fit beside the K double buffer in the histogram's space (dead
    // from here), they are copied once and every sweep reads them in place: no
    // list rebuild, copy or barrier per tile.
    constexpr int kResident = 2 + tau_region_bytes<E, D>(BINS) / (kBK * KS);
    // streaming sweeps: a ring over the same slots where tiles arrive by the
    // LDS copy engine (bf16, d = 128); register-staged tiles keep two buffers
    constexpr bool kDMA = sizeof(E) == 2 && D == 128;
    constexpr int kRing = kDMA ? (kResident < 4 ? kResident : 4) : 2;
    constexpr int kTileRowsPerWave = kBK / kWaves;   // copy instructions per wave and tile
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
      if (wave_busy && !dense) {
        // this sweep rewrites the wave's mask and its tiles above lo
        for (int e = lane; e < n_words; e += kWave) {
          mbits[w * n_words + e] = 0u;
          hbits[w * n_words + e] = 0u;
          hbits[(kWaves + w) * n_words + e] = 0u;
          lbits[w * n_words + e] = 0u;
        }
      }
      float F0 = 0, F1 = 0, F2 = 0, cnt = 0;
      // This wave's bits of the 32-tile word it is walking (final mask and tiles
      // above lo), kept in wave-uniform registers and written to LDS when the
      // walk leaves the word: an LDS write inside the tile loop would make the
      // wave wait for the next tile's copy in flight (the compiler cannot tell
      // the two LDS destinations apart), which would expose the copy's latency.
      // Tiles are listed in increasing order and a word never spans two list
      // chunks, so every word is written at most once per sweep.
      int bit_wd = -1;
      uint32_t m_word = 0u, l_word = 0u, h0_word = 0u, h1_word = 0u;
      auto flush_bits = [&]() {
        if (bit_wd >= 0 && lane == 0) {
          mbits[w * n_words + bit_wd] = m_word;
          hbits[w * n_words + bit_wd] = h0_word;
          hbits[(kWaves + w) * n_words + bit_wd] = h1_word;
          lbits[w * n_words + bit_wd] = l_word;
        }
        bit_wd = -1;
        m_word = l_word = h0_word = h1_word = 0u;
      };
      // f, f', f'' terms of key tile kt (staged at kl) and its mask bits
      auto sweep_tile = [&](int kt, const char* kl) {
        auto body = [&](auto masked) {
          const int lim = row_limit(kt * kBK, iq, N, P.causal, h);
          f32x16 acc[2];
          float cnt_at[3];
          cnt_at[0] = Ent<AK>::count(F0, F1, F2, cnt);
          tile_scores<E, D>(acc, kl, KS, qf, lane, lim, masked);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const float t = clamp01(fmaf(acc[kb][j], P.scale, -tau));
              Ent<AK>::sweep(t, P.beta, F0, F1, F2, cnt);
            }
            cnt_at[kb + 1] = Ent<AK>::count(F0, F1, F2, cnt);
          }
          if (!dense) {
            const bool any0 = __ballot(cnt_at[1] > cnt_at[0]) != 0ull;
            const bool any1 = __ballot(cnt_at[2] > cnt_at[1]) != 0ull;
            const bool any = any0 || any1;
            // does the tile hold a score above some row's lower bracket end?
            float mx = fmax_nan(acc[0][0], acc[1][0]);
#pragma unroll
            for (int j = 1; j < 16; ++j) mx = fmax_nan(mx, fmax_nan(acc[0][j], acc[1][j]));
            // (the ballot runs on every lane: it must see every row)
            const bool above = __ballot(fmaf(mx, P.scale, -lo) > 0.0f) != 0ull;
            const int wd = __builtin_amdgcn_readfirstlane(kt >> 5);
            if (wd != bit_wd) {
              flush_bits();
              bit_wd = wd;
            }
            if (any) m_word |= 1u << (kt & 31);
            if (any0) h0_word |= 1u << (kt & 31);
            if (any1) h1_word |= 1u << (kt & 31);
            if (above) l_word |= 1u << (kt & 31);
          }
        };
        if (wave_has_tail || (kt * kBK + kBK > N) || (P.causal && kt * kBK + kBK - 1 > wq0))
          body(std::true_type{});
        else
          body(std::false_type{});
      };
      if (n_res >= 0) {
        for (int i = 0; i < n_res; ++i)
          if (wave_busy && cand(w, list[i])) sweep_tile(list[i], slot(i));
        flush_bits();
      } else {
        for (int base = 0; base < kt_end; base += kChunk) {
          const int n = build_list(base, min(kChunk, kt_end - base), cand, list, wbits, flags, counter);
          RowTiles<E, D, kBK> st(Kh, N, w, lane);
          if constexpr (kRing > 2) {
            // Copy ring of kRing tile slots (the histogram's space holds two of
            // them): tile i sits in slot i % kRing and up to kRing - 1 copies are
            // in flight, so a copy has several tiles' work to land.  Nothing else
            // touches vector memory in this loop, so the wave's outstanding
            // copies are counted exactly.
#pragma unroll
            for (int j = 0; j < kRing - 1; ++j)
              if (j < n) st.fetch(slot(j), (base + list[j]) * kBK);
            for (int i = 0; i < n; ++i) {
              // tile i has landed once at most the copies of tiles i+1 .. are in flight
              const int ahead = min(kRing - 2, n - 1 - i);
              if (ahead >= 2) wait_vmcnt<2 * kTileRowsPerWave>();
              else if (ahead == 1) wait_vmcnt<kTileRowsPerWave>();
              else wait_vmcnt<0>();
              __builtin_amdgcn_s_barrier();   // every wave's part of tile i; slot of tile i-1 free
              if (i + kRing - 1 < n) st.fetch(slot((i + kRing - 1) % kRing), (base + list[i + kRing - 1]) * kBK);
              if (wave_busy && ((wbits[i] >> w) & 1)) sweep_tile(base + list[i], slot(i % kRing));
            }
            __syncthreads();
          } else {
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
          flush_bits();
        }
      }
      F0 += __shfl_xor(F0, 32);
      F1 += __shfl_xor(F1, 32);
      F2 += __shfl_xor(F2, 32);
      tau_step<AK>(F0, F1, F2, P.beta, P.mode, P.tol, max_iters, lo, hi, tau, conv, iters);
      // Candidates of the next sweep: tau only moves up from lo, so a tile with
      // no score above the lo this sweep used stays empty for every row; a wave
      // whose rows have all converged needs none.  (Only this wave's bits are
      // written; every reader of them passed a barrier since its last read.)
      if (wave_busy && !dense) {
        const bool busy_next = __ballot(!conv) != 0ull;
        for (int e = lane; e < n_words; e += kWave) cbits[w * n_words + e] = busy_next ? lbits[w * n_words + e] : 0u;
      }
    }

    // block_mask row of this wave from the final bits (every tile, so no zero fill)
    if (wave_rows) {
      for (int kt = lane; kt < P.n_kt; kt += kWave) {
        const uint32_t b = 1u << (kt & 31), e = (uint32_t)(kt >> 5);
        const bool m = mbits[w * n_words + e] & b;
        const uint32_t v = m ? (1u | ((hbits[w * n_words + e] & b) ? 2u : 0u) |
                                ((hbits[(kWaves + w) * n_words + e] & b) ? 4u : 0u))
                             : 0u;
        mrow[kt] = (uint8_t)v;
      }
    }
    if (valid && h == 0) {
      tau_out[(size_t)bh * P.ld + iq] = tau;
      if (iters_out) iters_out[(size_t)bh * P.ld + iq] = (uint8_t)min(iters, 255);
    }

    // ---- P V over the active tiles of the final mask (bf16).  Q is still in
    // registers, tau in a register and the mask in LDS; V tiles take the
    // histogram's place.
    if constexpr (kFusePV) {
      __syncthreads();   // every wave's final mask bits (and the histogram is dead)
      char* vbuf = reinterpret_cast<char*>(hist);                       // 2 x [64][KS]
      const E* Vh = V + (size_t)bh * P.ld * D;
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
      if (valid) store_out<D>(oacc, out, (size_t)bh * P.ld + iq, h, P.out_bf16 != 0);
    }
  };
  if constexpr (kFusePV) {
    // persistent (bf16): one workgroup per resident slot, units from the work queue
    __shared__ int s_unit;
    int bh, qtile;
    while (next_unit(queue, &s_unit, (N + kBQW - 1) / kBQW, Pk.BH, Pk.causal, bh, qtile)) {
      unit(bh, qtile);
      __syncthreads();   // the next unit reuses the LDS
    }
  } else {
    int bh, qtile;
    map_tile((N + kBQW - 1) / kBQW, Pk.BH, Pk.causal, bh, qtile);
    unit(bh, qtile);
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
  const E* Qh = Q + (size_t)bh * P.ld * D;
  const E* Kh = K + (size_t)bh * P.ld * D;
  const E* Vh = kTr ? Vsrc + (size_t)bh * P.ld * D : Vsrc + (size_t)bh * D * P.Np;

  char* kbuf = smem;                                 // 2 x [64][KS]
  char* vbuf = kbuf + 2 * kBK * KS;                  // 2 x V tile
  short* list = reinterpret_cast<short*>(vbuf + 2 * VT);
  uint8_t* wbits = reinterpret_cast<uint8_t*>(list + kChunk);
  uint8_t* flags = wbits + kChunk;
  int* counter = reinterpret_cast<int*>(flags + kChunk);

  Frag<E> qf[D / 16];
  load_qfrags<E, D>(qf, Qh + (size_t)iq * D, valid, h);
  const float tau = valid ? tau_in[(size_t)bh * P.ld + iq] : INFINITY;
  const bool wave_has_tail = wq0 + kBQ > N;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};

  const uint8_t* mrow0 = mask + (size_t)bh * P.mhs + (size_t)qtile * kWaves * P.mrs;
  auto active = [&](int ww, int kt) -> bool {
    return (qtile * kWaves + ww) < P.n_q32 && mrow0[(size_t)ww * P.mrs + kt] != 0;
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
  if (valid) store_out<D>(oacc, out, (size_t)bh * P.ld + iq, h, P.out_bf16 != 0);
}

// --------------------------------------------------------- transposes ---
// [BH][N][D] -> [BH][D][Np], zero for n in [N, Np).
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E* __restrict__ in, E* __restrict__ outp,
                                                   int N, int ld, int D, int Np) {
  __shared__ E t[64][65];
  const E* src = in + (size_t)blockIdx.z * ld * D;
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
  const size_t hoff = (size_t)bh * P.ld * D;
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
  const float tau = valid ? tau_in[(size_t)bh * P.ld + iq] : INFINITY;
  const bool wave_has_tail = wq0 + kBQ > N;

  f32x16 gacc[D / 32];                               // dQ, live in the second pass only
  float num = 0.0f, den = 0.0f, dlt = 0.0f;

  const uint8_t* mrow0 = mask + (size_t)bh * P.mhs + (size_t)qtile * kWaves * P.mrs;
  // the wave's mask byte of tile kt (0 past the last query block)
  auto mbyte = [&](int ww, int kt) -> uint32_t {
    return (qtile * kWaves + ww) < P.n_q32 ? (uint32_t)mrow0[(size_t)ww * P.mrs + kt] : 0u;
  };
  // two bits per wave: which 32-key halves of the tile hold a probability
  auto halves = [&](int ww, int kt) -> uint32_t { return half_bits(mbyte(ww, kt)); };
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
                          : build_list<2>(base, min(kChunk, P.n_kt - base), halves, list, wbits, flags, counter);
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
        const uint32_t hv = (wbits[i] >> (2 * w)) & 3u;   // this wave's live halves
        if (hv) {
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
              if (!((hv >> kb) & 1u)) continue;   // no probability in this 32x32 micro-tile
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
                  Frag<E> kf[D / 32];
                  if constexpr (kTr) {
                    ld_col8_row<D / 32, true>(kf, kl, KS, koff, lane);
                  } else {
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                      const E* krow = reinterpret_cast<const E*>(tl + (32 * db + c32) * VS);
                      ld4x2(kf[db], krow + koff, krow + koff + 8);
                    }
                  }
#pragma unroll
                  for (int db = 0; db < D / 32; ++db) {
                    mma(gacc[db], kf[db], sf);
                    if constexpr (kNeedsLo<E>) mma(gacc[db], kf[db], sl);
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
      for (int ww = 0; ww < kWaves; ++ww) word |= mbyte(ww, kt) << (8 * ww);
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
  const size_t hoff = (size_t)bh * P.ld * D;
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
  // waves 0, 1 cover the two 32-key halves of key tile A, waves 2, 3 those of
  // key tile B: a wave's work is one 32x32 micro-tile per query block, live
  // when the mask byte's bit for its half is set.  The transposed mask gives
  // each key tile's query rows contiguously.
  auto active = [&](int ww, int r) -> bool {
    const int kt = ww < 2 ? ktA : ktB;
    if (kt >= P.n_kt || (ktile * 128 + 32 * ww) >= N) return false;
    return (half_bits(maskT[((size_t)bh * P.n_kt + kt) * np + r]) >> (ww & 1)) & 1u;
  };

  RowTiles<E, D, kBQ> sq(Q + hoff, N, w, lane), so(dO + hoff, N, w, lane);
  ColStage<E, D, kBQ> sqt, sot;
  // per-query tau and delta of a block: copy engine (waves 0 and 1, 32 lanes
  // each; rows past N read as zeros and are masked by the row limits) or
  // registers of the first 32 threads
  __amdgpu_buffer_rsrc_t rs_td = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(w == 0 ? tau_in + (size_t)bh * P.ld : delta_in + (size_t)bh * N), (short)0, N * 4,
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
        sta = qi < N ? tau_in[(size_t)bh * P.ld + qi] : INFINITY;
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
        [[maybe_unused]] double sd[kTr ? 1 : 16] = {};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          Frag<E> a, b;
          ld8(a, reinterpret_cast<const E*>(qtl + c32 * KS) + 16 * c + 8 * h);
          if constexpr (kDirect) {
            Frag<E> kc;
            ld8(kc, reinterpret_cast<const E*>(klds + (32 * w + c32) * KS) + 16 * c + 8 * h);
            mma(sacc, a, kc);
          } else if constexpr (!kTr) {
            mma_chunk64(sd, a, kf[c]);
          } else {
            mma(sacc, a, kf[c]);
          }
          ld8(b, reinterpret_cast<const E*>(otl + c32 * KS) + 16 * c + 8 * h);
          mma(pacc, b, vf[c]);
        }
        if constexpr (!kTr) round_acc(sacc, sd);
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
          // dK = sum_i dS_ij q_i: the queries of a cluster are nearly parallel
          // and large, so the bf16 rounding of dS alone would cost about the
          // whole stated tolerance on some keys' rows; dS goes in as a hi/lo
          // bf16 pair, as in the dQ kernel.
          Frag<E> pf, sf, sl;
          from_acc(pf, sacc, 8 * s);
          split_acc(sf, sl, pacc, 8 * s);
          const int qoff = 16 * s + 4 * h;
          Frag<E> ob[D / 32], qb[D / 32];
          if constexpr (kTr) {
            ld_col8_row<D / 32, false>(ob, otl, KS, qoff, lane);
            ld_col8_row<D / 32, false>(qb, qtl, KS, qoff, lane);
          } else {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const E* orow = reinterpret_cast<const E*>(ottl + (32 * db + c32) * TS);
              const E* qrow = reinterpret_cast<const E*>(qttl + (32 * db + c32) * TS);
              ld4x2(ob[db], orow + qoff, orow + qoff + 8);
              ld4x2(qb[db], qrow + qoff, qrow + qoff + 8);
            }
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            mma(dva[db], pf, ob[db]);
            mma(dka[db], sf, qb[db]);
            if constexpr (kNeedsLo<E>) mma(dka[db], sl, qb[db]);
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

// ------------------------------------------------------- k_entmax_rows ---
// alpha-entmax of materialised score rows (no attention): x = (alpha-1) s,
// tau per row, p = [x - tau]_+^(1/(alpha-1)) ("AdaSplash: Adaptive Sparse
// Flash Attention", "Accelerated Alpha-Entmax Transformation": the transform
// on its own, where Halley-bisection replaces plain bisection).  One wave per
// row: lane l holds elements 4 (l + 64 c) .. +3 for chunks c, in registers
// when the row has at most 64 T elements (T > 0), else read again from memory
// by every sweep (T = 0).  Sweep sums are reduced across the wave with DPP and
// lane permutes, so no barrier is involved; the histogram is the wave's own
// in LDS.  -inf scores are masked entries (p = 0, not counted in n).
struct RowParams {
  long long rows;
  int n, mode, max_iters, hshift, vec;
  float scale, beta, alpha, tol;
};
constexpr int kRowBins = 16;

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) { return v + dpp_f<CTRL>(v); }
// sum over the whole wave, the same on every lane (fixed order: deterministic)
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = half_max32(v);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename E>
__device__ __forceinline__ f32x4 load4(const E* row, int e, int n, bool vec) {
  f32x4 r = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (vec && e + 3 < n) {
    if constexpr (sizeof(E) == 4) {
      r = *reinterpret_cast<const f32x4*>(row + e);
    } else {
      const bf16x4 b = *reinterpret_cast<const bf16x4*>(row + e);
      r = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e + i < n) r[i] = (float)row[e + i];
  }
  return r;
}
template <typename E>
__device__ __forceinline__ void store4(E* row, int e, int n, bool vec, const f32x4& v) {
  if (vec && e + 3 < n) {
    if constexpr (sizeof(E) == 4) {
      *reinterpret_cast<f32x4*>(row + e) = v;
    } else {
      *reinterpret_cast<bf16x4*>(row + e) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e + i < n) row[e + i] = (E)v[i];
  }
}

template <typename EI, typename EO, int AK, int T>
__global__ __launch_bounds__(kThreads) void k_entmax_rows(const EI* __restrict__ S, EO* __restrict__ Pout,
                                                          float* __restrict__ tau_out,
                                                          uint8_t* __restrict__ iters_out, RowParams P) {
  __shared__ unsigned long long hist_all[kWaves][2 * kRowBins];
  constexpr int NC = T > 0 ? T / 4 : 1;      // register chunks per lane
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = P.n;
  const bool vec = P.vec != 0;
  const int n_chunks = (n + 255) / 256;      // chunks of 256 elements (4 per lane)
  unsigned long long* hr = hist_all[w];

  for (long long r = (long long)blockIdx.x * kWaves + w; r < P.rows; r += (long long)gridDim.x * kWaves) {
    const EI* row = S + r * n;
    f32x4 xr[NC];
    // the row's x values in registers (T > 0), its maximum and its count
    float m = -INFINITY, cnt = 0.0f;
    auto for_chunks = [&](auto&& fn) {
      if constexpr (T > 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) fn(xr[c], 4 * (lane + 64 * c));
      } else {
        for (int c = 0; c < n_chunks; ++c) {
          const int e = 4 * (lane + 64 * c);
          f32x4 v = load4(row, e, n, vec) * P.scale;
          fn(v, e);
        }
      }
    };
    if constexpr (T > 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) xr[c] = load4(row, 4 * (lane + 64 * c), n, vec) * P.scale;
    }
    for_chunks([&](const f32x4& v, int) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = fmax_nan(m, v[i]);
        cnt += v[i] > -INFINITY ? 1.0f : 0.0f;
      }
    });
    const float xmax = wave_max(m);
    const float nv = wave_sum(cnt);
    // bracket [max x - 1, max x - n^(1-alpha)], rounded outward
    float lo = 0.0f, hi = 0.0f, tau = 0.0f;
    const bool empty = !(nv > 0.0f);
    if (!empty) {
      const double dl = (double)xmax - 1.0;
      lo = (float)dl;
      if ((double)lo > dl) lo = nextafterf(lo, -INFINITY);
      const double dh = (double)xmax - pow((double)nv, 1.0 - (double)P.alpha);
      hi = (float)dh;
      if ((double)hi < dh) hi = nextafterf(hi, INFINITY);
      if (hi < lo) hi = lo;
    }
    if (P.mode == EA_TAU_HIST_HALLEY && !empty) {
      for (int e = lane; e < 2 * kRowBins; e += kWave) hr[e] = 0ull;
      __builtin_amdgcn_wave_barrier();
      const float width = fmaxf(hi - lo, 1e-30f);
      const float bin_scale = (float)kRowBins / width;
      const float ysc = (float)((1u << P.hshift) - 1u);
      for_chunks([&](const f32x4& v, int) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hist_add<false>(0u, hr, clamp01(v[i] - lo), bin_scale, ysc, kRowBins);
      });
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      hist_start<AK, kRowBins>(hr, width, xmax, P.hshift, P.beta, lo, hi, tau);
    } else if (P.mode == EA_TAU_HALLEY_BISECT) {
      tau = lo;
    } else {
      tau = 0.5f * (lo + hi);
    }
    // refinement sweeps: the same stopping rules as the attention kernel
    bool conv = empty;
    int iters = 0;
    while (!conv) {
      float F0 = 0, F1 = 0, F2 = 0, c2 = 0;
      for_chunks([&](const f32x4& v, int) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Ent<AK>::sweep(clamp01(v[i] - tau), P.beta, F0, F1, F2, c2);
      });
      F0 = wave_sum(F0);
      F1 = wave_sum(F1);
      if (P.mode != EA_TAU_BISECT && AK != AK20) F2 = wave_sum(F2);
      tau_step<AK>(F0, F1, F2, P.beta, P.mode, P.tol, P.max_iters, lo, hi, tau, conv, iters);
    }
    // probabilities at the final tau
    EO* prow = Pout + r * n;
    const float ptau = empty ? INFINITY : tau;
    for_chunks([&](const f32x4& v, int e) {
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pp, u;
        Ent<AK>::pu(clamp01(v[i] - ptau), P.beta, pp, u);
        o[i] = pp;
      }
      store4(prow, e, n, vec, o);
    });
    if (lane == 0) {
      tau_out[r] = empty ? INFINITY : tau;
      if (iters_out) iters_out[r] = (uint8_t)min(iters, 255);
    }
  }
}

// ------------------------------------------------------------ padding ---
// Variable-length calls: each batch b sees only its first L keys and query
// rows.  A query row past L sees no key at all: its output row is 0, tau is
// +inf (so every p = [x - tau]_+^beta is 0) and its sweep count 0; keys past L
// get zero dK and dV, rows past L zero dQ, and every block-mask entry outside
// the batch's [ceil(L/32)] x [ceil(L/64)] tiles is 0.  These kernels write
// exactly those entries of one batch (all H heads) with plain stores.
template <typename EO>
__global__ __launch_bounds__(256) void k_pad_fwd(EO* __restrict__ out, float* __restrict__ tau,
                                                 uint8_t* __restrict__ iters, uint8_t* __restrict__ mask,
                                                 int H, int N, int L, int D, int n_q32, int n_kt, int n_q32L,
                                                 int n_ktL) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long t0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long rows = (long long)H * (N - L);
  for (long long e = t0; e < rows * D; e += stride) {
    const long long r = e / D, h = r / (N - L), i = L + r % (N - L);
    out[((size_t)h * N + i) * D + e % D] = (EO)0.0f;
  }
  for (long long r = t0; r < rows; r += stride) {
    const long long h = r / (N - L), i = L + r % (N - L);
    tau[(size_t)h * N + i] = INFINITY;
    if (iters) iters[(size_t)h * N + i] = 0;
  }
  const long long me = (long long)H * n_q32 * n_kt;
  for (long long e = t0; e < me; e += stride) {
    const long long kt = e % n_kt, r = (e / n_kt) % n_q32;
    if (r >= n_q32L || kt >= n_ktL) mask[e] = 0;
  }
}
template <typename EO>
__global__ __launch_bounds__(256) void k_pad_bwd(EO* __restrict__ dq, EO* __restrict__ dk, EO* __restrict__ dv,
                                                 int H, int N, int L, int D) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long n = (long long)H * (N - L) * D;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    const long long r = e / D, h = r / (N - L), i = L + r % (N - L);
    const size_t off = ((size_t)h * N + i) * D + e % D;
    dq[off] = (EO)0.0f;
    dk[off] = (EO)0.0f;
    dv[off] = (EO)0.0f;
  }
}

// =============================================================== host ===

struct Shape {
  int B, H, N, d, esz, n_kt, n_q32, n_qt128, n_qt256, n_kt128, Np;
  int BH;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kMaxN = 1 << 20;

Shape shape_of(int B, int H, int N, int d, int esz) {
  Shape s;
  s.B = B;
  s.H = H;
  s.N = N;
  s.d = d;
  s.esz = esz;
  s.n_kt = (N + kBK - 1) / kBK;
  s.n_q32 = (N + kBQ - 1) / kBQ;
  s.n_qt128 = (N + kBQW - 1) / kBQW;
  s.n_qt256 = (N + 255) / 256;
  s.n_kt128 = (N + 127) / 128;
  s.Np = s.n_kt * kBK;
  s.BH = B * H;
  return s;
}

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
  if (desc->key_lens) {
    for (int b = 0; b < desc->B; ++b)
      if (desc->key_lens[b] < 0 || desc->key_lens[b] > desc->N) return EA_ERR_SHAPE;
  }
  if (s) *s = shape_of(desc->B, desc->H, desc->N, desc->d, desc->in_dtype == EA_BF16 ? 2 : 4);
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
// one byte per (32-query block, 64-key tile), rows padded to 64 tiles: the
// size of the block mask, about N^2 / 2048 bytes per head
size_t blkcode_bytes(const Shape& s) {
  return align_up((size_t)s.BH * s.n_q32 * (size_t)blk_row(s.n_kt), 256);
}

// the block mask transposed, [BH][n_kt][n_q32 rounded up to 4] bytes
size_t maskt_bytes(const Shape& s) {
  return align_up((size_t)s.BH * s.n_kt * (size_t)((s.n_q32 + 3) & ~3), 256);
}

size_t workspace_bytes(const Shape& s) {
  // forward: [V^T] | row maxima | block codes | work queues;
  // backward: [K^T | Q^T | dO^T] | delta | transposed mask
  const size_t fwd = transposed_bytes(s) + row_bytes(s) + blkcode_bytes(s) + kQueueBytes;
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

// Fixed-point bits S of the histogram moments: N (2^(40-S) - 1) < 2^40 and
// N (2^S - 1)^2 < 2^64 for every N <= 2^20; S = 24 up to N = 65536.
int hist_shift(int N) {
  int L = 1;
  while ((1 << L) < N) ++L;
  return L <= 16 ? 24 : 40 - L;
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
  P.hshift = hist_shift(s.N);
  P.ld = s.N;
  P.mrs = s.n_kt;
  P.mhs = (long long)s.n_q32 * s.n_kt;
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
  // resident row-max workgroups: two waves per SIMD, 64 queries per wave
  const long tiles = (long)((s.N + kRowmaxQ - 1) / kRowmaxQ) * s.BH, slots = 8L * cus / kRowmaxWaves;
  return 2 * tiles > 3 * slots && 2 * tiles <= 5 * slots;
}

// Workgroups of a persistent kernel (next_unit): as many as stay resident at
// once (the occupancy for its LDS size, times the compute units), at most
// one per unit; a multiple of 8 when there is one queue per XCD, so that
// every queue has workgroups on its XCD.
int persistent_grid(const void* fn, size_t lds, int units, int BH) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess || per_cu <= 0)
    per_cu = 1, cus = 64;
  int g = cus * per_cu;
  if (g > units) g = units;
  if ((BH & 7) == 0) g = (g + 7) & ~7;   // units is then a multiple of 8 too
  return g > 0 ? g : 1;
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

// Dynamic LDS above the default 64 KB must be allowed per kernel before its
// first launch.
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

// Launches kernel k and returns the launch's own status (an error left by an
// earlier, unrelated HIP call is neither reported nor cleared).
template <typename... KA, typename... CA>
int launch(void (*k)(KA...), dim3 grid, dim3 block, size_t lds, hipStream_t st, CA... args) {
  auto go = [&](KA... a) {
    void* argv[] = {static_cast<void*>(&a)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, lds, st);
  };
  return go(args...) == hipSuccess ? EA_OK : EA_ERR_LAUNCH;
}

template <typename E, int D, int AK>
int launch_fwd(const Shape& s, Params P, const void* q, const void* k, const void* v, void* out,
               float* tau, uint8_t* mask, uint8_t* iters, void* ws, hipStream_t st, StageTimer tm) {
  constexpr bool kTr = sizeof(E) == 2;
  constexpr int KS = row_stride<E, D>();
  constexpr int BINS = 16;
  const E* Q = static_cast<const E*>(q);
  const E* K = static_cast<const E*>(k);
  const E* V = static_cast<const E*>(v);
  if (s.N == 0) return EA_OK;
  char* w = static_cast<char*>(ws);
  E* Vt = reinterpret_cast<E*>(w);
  float* rowmax = reinterpret_cast<float*>(w + transposed_bytes(s));
  uint8_t* blkc = reinterpret_cast<uint8_t*>(w + transposed_bytes(s) + row_bytes(s));
  int* queue = reinterpret_cast<int*>(w + transposed_bytes(s) + row_bytes(s) + blkcode_bytes(s));

  // every LDS size is checked and allowed before anything is enqueued
  const size_t rm_lds = kTr ? (size_t)2 * kRowmaxTPS * DirectTile<D>::BYTES : (size_t)2 * kBK * KS;
  const size_t tau_lds = (size_t)2 * kBK * KS + (size_t)tau_region_bytes<E, D>(BINS) + 4 * kChunk +
                         (size_t)5 * kWaves * ((s.n_kt + 31) / 32) * 4 + 64;
  constexpr int VT = D * (kBK * (int)sizeof(E) + 16);
  const size_t pv_lds = (size_t)2 * kBK * KS + (size_t)2 * VT + 4 * kChunk + 16;
  auto ktau = k_tau<E, D, AK, BINS>;
  auto kpv = k_pv<E, D, AK>;
  int rc;
  if constexpr (kTr) {
    if ((rc = set_lds(k_rowmax16<D>, rm_lds)) != EA_OK) return rc;
  } else {
    if ((rc = set_lds(k_rowmax<E, D>, rm_lds)) != EA_OK) return rc;
    if ((rc = set_lds(kpv, pv_lds)) != EA_OK) return rc;
  }
  if ((rc = set_lds(ktau, tau_lds)) != EA_OK) return rc;

  tm.begin(EA_STAGE_FWD_PREP);
  if constexpr (!kTr) {
    if ((rc = launch(k_transpose<E>, dim3(s.Np / 64, D / 64, s.BH), dim3(256), 0, st, V, Vt, s.N, P.ld, D, s.Np)) != EA_OK)
      return rc;
  }
  tm.end(EA_STAGE_FWD_PREP);

  tm.begin(EA_STAGE_ROWMAX);
  if constexpr (kTr) {
    P.pair_qt = pair_query_tiles(s, P.causal) ? 1 : 0;
    const int n_qt = (s.N + kRowmaxQ - 1) / kRowmaxQ;
    const int units = P.pair_qt ? (n_qt + 1) / 2 : n_qt;
    rc = launch(k_rowmax16<D>, dim3(units * s.BH), dim3(64 * kRowmaxWaves), rm_lds, st, Q, K, P, rowmax, blkc,
                queue);
  } else {
    rc = launch(k_rowmax<E, D>, dim3(s.n_qt256 * s.BH), dim3(kThreads), rm_lds, st, Q, K, P, rowmax, blkc,
                queue);
  }
  if (rc != EA_OK) return rc;
  tm.end(EA_STAGE_ROWMAX);

  const dim3 g(s.n_qt128 * s.BH);
  tm.begin(EA_STAGE_TAU);   // bf16: tau, block mask and P V in one kernel
  // bf16: persistent workgroups (next_unit)
  const dim3 gp(kTr ? persistent_grid(reinterpret_cast<const void*>(ktau), tau_lds, s.n_qt128 * s.BH, s.BH)
                    : s.n_qt128 * s.BH);
  if ((rc = launch(ktau, gp, dim3(kThreads), tau_lds, st, Q, K, V, (const float*)rowmax, (const uint8_t*)blkc, P,
                   tau, mask, iters, out, queue)) != EA_OK)
    return rc;
  tm.end(EA_STAGE_TAU);

  tm.begin(EA_STAGE_PV);   // empty for bf16 (fused above)
  if constexpr (!kTr) {
    if ((rc = launch(kpv, g, dim3(kThreads), pv_lds, st, Q, K, (const E*)Vt, (const float*)tau,
                     (const uint8_t*)mask, P, out)) != EA_OK)
      return rc;
  }
  tm.end(EA_STAGE_PV);
  return EA_OK;
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

  constexpr int KS = row_stride<E, D>();
  constexpr int TT = kTr ? 0 : D * (kBK * (int)sizeof(E) + 16);
  constexpr int NB = (2 * (2 * kBK * KS + TT) + 4 * kChunk + 16) <= 160 * 1024 ? 2 : 1;
  const size_t dq_lds = (size_t)NB * (2 * kBK * KS + TT) + 4 * kChunk + 16;
  const size_t kv_lds = (size_t)kv_stages<E, D>() * kv_step_bytes<E, D>() + 4 * kChunk + 16 +
                        (kTr && D == 128 ? (size_t)4 * kBQ * KS : 0);   // the K rows (bf16, d = 128)
  auto kdq = k_bwd_dq<E, D, AK, NB>;
  auto kkv = k_bwd_dkdv<E, D, AK>;
  int rc;
  if ((rc = set_lds(kdq, dq_lds)) != EA_OK) return rc;
  if ((rc = set_lds(kkv, kv_lds)) != EA_OK) return rc;

  tm.begin(EA_STAGE_BWD_PREP);
  if constexpr (!kTr) {
    const dim3 tg(s.Np / 64, D / 64, s.BH);
    if ((rc = launch(k_transpose<E>, tg, dim3(256), 0, st, K, Kt, s.N, P.ld, D, s.Np)) != EA_OK) return rc;
    if ((rc = launch(k_transpose<E>, tg, dim3(256), 0, st, Q, Qt, s.N, P.ld, D, s.Np)) != EA_OK) return rc;
    if ((rc = launch(k_transpose<E>, tg, dim3(256), 0, st, dO, dOt, s.N, P.ld, D, s.Np)) != EA_OK) return rc;
  }
  tm.end(EA_STAGE_BWD_PREP);

  tm.begin(EA_STAGE_DQ);
  if ((rc = launch(kdq, dim3(s.n_qt128 * s.BH), dim3(kThreads), dq_lds, st, Q, K, V, dO, (const E*)Kt, tau,
                   mask, P, delta, maskT, dq)) != EA_OK)
    return rc;
  tm.end(EA_STAGE_DQ);

  tm.begin(EA_STAGE_DKDV);
  if ((rc = launch(kkv, dim3(s.n_kt128 * s.BH), dim3(kThreads), kv_lds, st, Q, K, V, dO, (const E*)Qt,
                   (const E*)dOt, tau, (const float*)delta, (const uint8_t*)maskT, P, dk, dv)) != EA_OK)
    return rc;
  tm.end(EA_STAGE_DKDV);
  return EA_OK;
}

// ------------------------------------------------- row transform host ---
int check_rows_desc(const ea_rows_desc* d) {
  if (!d) return EA_ERR_NULL;
  if (d->rows < 0 || d->n < 1 || d->n > kMaxN || d->rows > ((long long)1 << 40) / d->n) return EA_ERR_SHAPE;
  if ((d->in_dtype != EA_F32 && d->in_dtype != EA_BF16) || (d->out_dtype != EA_F32 && d->out_dtype != EA_BF16))
    return EA_ERR_DTYPE;
  if (d->tau_mode < EA_TAU_HIST_HALLEY || d->tau_mode > EA_TAU_BISECT) return EA_ERR_UNSUPPORTED;
  if (d->max_iters < 0 || d->max_iters > 250) return EA_ERR_UNSUPPORTED;
  if (!(d->tol >= 0.0f) || !(d->tol < 1.0f)) return EA_ERR_UNSUPPORTED;
  return EA_OK;
}

template <typename EI, typename EO, int AK>
int launch_rows(const ea_rows_desc* d, RowParams P, const void* s, void* p, float* tau, uint8_t* iters,
                hipStream_t st) {
  if (d->rows == 0) return EA_OK;
  const long long groups = (d->rows + kWaves - 1) / kWaves;
  const dim3 g((unsigned)(groups < 8192 ? groups : 8192));
  const EI* S = static_cast<const EI*>(s);
  EO* Po = static_cast<EO*>(p);
  if (d->n <= 1024) return launch(k_entmax_rows<EI, EO, AK, 16>, g, dim3(kThreads), 0, st, S, Po, tau, iters, P);
  if (d->n <= 4096) return launch(k_entmax_rows<EI, EO, AK, 64>, g, dim3(kThreads), 0, st, S, Po, tau, iters, P);
  return launch(k_entmax_rows<EI, EO, AK, 0>, g, dim3(kThreads), 0, st, S, Po, tau, iters, P);
}

template <typename EI, typename EO>
int dispatch_rows_ak(float alpha, const ea_rows_desc* d, RowParams P, const void* s, void* p, float* tau,
                     uint8_t* iters, hipStream_t st) {
  switch (alpha_kind(alpha)) {
    case AK15: return launch_rows<EI, EO, AK15>(d, P, s, p, tau, iters, st);
    case AK20: return launch_rows<EI, EO, AK20>(d, P, s, p, tau, iters, st);
    case AK125: return launch_rows<EI, EO, AK125>(d, P, s, p, tau, iters, st);
    default: return launch_rows<EI, EO, AKGEN>(d, P, s, p, tau, iters, st);
  }
}

// ------------------------------------------------ no-allocation forward ---
// entmax_attn_fwd_static runs the forward on a fixed-size file-scope device
// array instead of a caller workspace.  Every GPU the library runs on holds
// its own copy of the array until the process ends.  In host code the array's
// name is not a device address: the address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that pointer is
// passed to kernels.  Calls on one GPU share the array, so overlapping calls
// there race; the forward writes every workspace byte it later reads, so
// nothing needs clearing between calls.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return EA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EA_OK;
}

// forward part of the workspace: [V^T] | row maxima | block codes | work queues
size_t fwd_workspace_bytes(const Shape& s) {
  return transposed_bytes(s) + row_bytes(s) + blkcode_bytes(s) + kQueueBytes;
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

int run_fwd(const Shape& s, const Params& P, const ea_desc* desc, float alpha, const void* q, const void* k,
            const void* v, void* out, float* tau, uint8_t* block_mask, uint8_t* tau_iters, void* ws,
            hipStream_t hs, StageTimer tm) {
  EA_DISPATCH(launch_fwd, s, P, q, k, v, out, tau, block_mask, tau_iters, ws, hs, tm);
}
int run_bwd(const Shape& s, const Params& P, const ea_desc* desc, float alpha, const void* q, const void* k,
            const void* v, const void* dout, const float* tau, const uint8_t* block_mask, void* dq, void* dk,
            void* dv, void* ws, hipStream_t hs, StageTimer tm) {
  EA_DISPATCH(launch_bwd, s, P, q, k, v, dout, tau, block_mask, dq, dk, dv, ws, hs, tm);
}

unsigned pad_grid(long long n) { return (unsigned)std::min<long long>(std::max<long long>((n + 255) / 256, 1), 4096); }

// The whole forward: one problem, or with key_lens one problem per batch on
// the same tensors (row stride N, mask strides of the full shape) followed by
// the padding of that batch.  Stage events are recorded for one problem only.
int forward_all(const Shape& s, const ea_desc* desc, float alpha, int causal, const void* q, const void* k,
                const void* v, void* out, float* tau, uint8_t* block_mask, uint8_t* tau_iters, void* ws,
                hipStream_t hs) {
  if (!desc->key_lens) {
    return run_fwd(s, make_params(desc, s, alpha, causal), desc, alpha, q, k, v, out, tau, block_mask, tau_iters,
                   ws, hs, StageTimer{desc->events, hs});
  }
  const size_t hrow = (size_t)s.H * s.N;                   // rows per batch
  const size_t ie = s.esz, oe = desc->out_dtype == EA_BF16 ? 2 : 4;
  const size_t mb = (size_t)s.H * s.n_q32 * s.n_kt;          // mask bytes per batch
  for (int b = 0; b < s.B; ++b) {
    const int L = desc->key_lens[b];
    const Shape sb = shape_of(1, s.H, L, s.d, s.esz);
    Params P = make_params(desc, sb, alpha, causal);
    P.ld = s.N;
    P.mrs = s.n_kt;
    P.mhs = (long long)s.n_q32 * s.n_kt;
    const size_t off = (size_t)b * hrow * s.d;
    char* ob = static_cast<char*>(out) + off * oe;
    uint8_t* mkb = block_mask + b * mb;
    float* tb = tau + b * hrow;
    uint8_t* ib = tau_iters ? tau_iters + b * hrow : nullptr;
    int rc = run_fwd(sb, P, desc, alpha, static_cast<const char*>(q) + off * ie, static_cast<const char*>(k) + off * ie,
                     static_cast<const char*>(v) + off * ie, ob, tb, mkb, ib, ws, hs, StageTimer{nullptr, hs});
    if (rc != EA_OK) return rc;
    const dim3 g(pad_grid((long long)s.H * std::max(s.N - L, 1) * s.d + (long long)mb));
    const int nq = (L + kBQ - 1) / kBQ, nk = (L + kBK - 1) / kBK;
    if (oe == 2)
      rc = launch(k_pad_fwd<__bf16>, g, dim3(256), 0, hs, reinterpret_cast<__bf16*>(ob), tb, ib, mkb, s.H, s.N, L,
                  s.d, s.n_q32, s.n_kt, nq, nk);
    else
      rc = launch(k_pad_fwd<float>, g, dim3(256), 0, hs, reinterpret_cast<float*>(ob), tb, ib, mkb, s.H, s.N, L,
                  s.d, s.n_q32, s.n_kt, nq, nk);
    if (rc != EA_OK) return rc;
  }
  return EA_OK;
}

int backward_all(const Shape& s, const ea_desc* desc, float alpha, int causal, const void* q, const void* k,
                 const void* v, const void* dout, const float* tau, const uint8_t* block_mask, void* dq, void* dk,
                 void* dv, void* ws, hipStream_t hs) {
  if (!desc->key_lens) {
    return run_bwd(s, make_params(desc, s, alpha, causal), desc, alpha, q, k, v, dout, tau, block_mask, dq, dk, dv,
                   ws, hs, StageTimer{desc->events, hs});
  }
  const size_t hrow = (size_t)s.H * s.N;
  const size_t ie = s.esz, oe = desc->out_dtype == EA_BF16 ? 2 : 4;
  const size_t mb = (size_t)s.H * s.n_q32 * s.n_kt;
  for (int b = 0; b < s.B; ++b) {
    const int L = desc->key_lens[b];
    const Shape sb = shape_of(1, s.H, L, s.d, s.esz);
    Params P = make_params(desc, sb, alpha, causal);
    P.ld = s.N;
    P.mrs = s.n_kt;
    P.mhs = (long long)s.n_q32 * s.n_kt;
    const size_t off = (size_t)b * hrow * s.d;
    char* qb = static_cast<char*>(dq) + off * oe;
    char* kb = static_cast<char*>(dk) + off * oe;
    char* vb = static_cast<char*>(dv) + off * oe;
    int rc = run_bwd(sb, P, desc, alpha, static_cast<const char*>(q) + off * ie, static_cast<const char*>(k) + off * ie,
                     static_cast<const char*>(v) + off * ie, static_cast<const char*>(dout) + off * ie,
                     tau + b * hrow, block_mask + b * mb, qb, kb, vb, ws, hs, StageTimer{nullptr, hs});
    if (rc != EA_OK) return rc;
    if (L < s.N) {
      const dim3 g(pad_grid((long long)s.H * (s.N - L) * s.d));
      if (oe == 2)
        rc = launch(k_pad_bwd<__bf16>, g, dim3(256), 0, hs, reinterpret_cast<__bf16*>(qb), reinterpret_cast<__bf16*>(kb),
                    reinterpret_cast<__bf16*>(vb), s.H, s.N, L, s.d);
      else
        rc = launch(k_pad_bwd<float>, g, dim3(256), 0, hs, reinterpret_cast<float*>(qb), reinterpret_cast<float*>(kb),
                    reinterpret_cast<float*>(vb), s.H, s.N, L, s.d);
      if (rc != EA_OK) return rc;
    }
  }
  return EA_OK;
}

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
  return forward_all(s, desc, alpha, causal, q, k, v, out, tau, block_mask, tau_iters, ws,
                     static_cast<hipStream_t>(stream));
}

int entmax_attn_fwd_static(const void* q, const void* k, const void* v, float alpha, int causal, void* out,
                           float* tau, uint8_t* block_mask, uint8_t* tau_iters, const ea_desc* desc,
                           void* stream) {
  Shape s;
  int st = check_desc(desc, &s);
  if (st != EA_OK) return st;
  if ((st = check_alpha(alpha)) != EA_OK) return st;
  if (causal != 0 && causal != 1) return EA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (s.N > 0) {
    if (!q || !k || !v || !out || !tau || !block_mask) return EA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(tau))
      return EA_ERR_ALIGN;
    if (fwd_workspace_bytes(s) > kStaticScratchBytes) return EA_ERR_WORKSPACE;
    if ((st = static_scratch(&ws)) != EA_OK) return st;
  }
  return forward_all(s, desc, alpha, causal, q, k, v, out, tau, block_mask, tau_iters, ws,
                     static_cast<hipStream_t>(stream));
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
  return backward_all(s, desc, alpha, causal, q, k, v, dout, tau, block_mask, dq, dk, dv, ws,
                      static_cast<hipStream_t>(stream));
}

int entmax_rows(const void* s, float alpha, void* p, float* tau, uint8_t* tau_iters, const ea_rows_desc* desc,
                void* stream) {
  int st = check_rows_desc(desc);
  if (st != EA_OK) return st;
  if ((st = check_alpha(alpha)) != EA_OK) return st;
  if (desc->rows > 0) {
    if (!s || !p || !tau) return EA_ERR_NULL;
    if (misaligned(s) || misaligned(p) || misaligned(tau)) return EA_ERR_ALIGN;
  }
  RowParams P;
  P.rows = desc->rows;
  P.n = desc->n;
  P.mode = desc->tau_mode;
  P.max_iters = desc->max_iters > 0 ? desc->max_iters : (desc->tau_mode == EA_TAU_BISECT ? 40 : 12);
  P.hshift = hist_shift(desc->n);
  P.vec = desc->n % 4 == 0 ? 1 : 0;
  P.alpha = alpha;
  P.scale = (float)((double)alpha - 1.0);
  P.beta = (float)(1.0 / ((double)alpha - 1.0));
  P.tol = desc->tol > 0.0f ? desc->tol : 1e-6f;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool ib = desc->in_dtype == EA_BF16, ob = desc->out_dtype == EA_BF16;
  if (ib && ob) return dispatch_rows_ak<__bf16, __bf16>(alpha, desc, P, s, p, tau, tau_iters, hs);
  if (ib) return dispatch_rows_ak<__bf16, float>(alpha, desc, P, s, p, tau, tau_iters, hs);
  if (ob) return dispatch_rows_ak<float, __bf16>(alpha, desc, P, s, p, tau, tau_iters, hs);
  return dispatch_rows_ak<float, float>(alpha, desc, P, s, p, tau, tau_iters, hs);
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
