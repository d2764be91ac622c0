// flare.hip -- gfx950 kernels and C ABI of the FLARE / FLARE++ routing forward.
//
// The method ("FLARE++: Low-rank attention with attention-synthesized
// routing"): FLARE encodes N tokens into M latents with one softmax-attention
// call whose queries are M latent queries (softmax over the tokens), then
// decodes every token with a second call whose queries are the token keys and
// whose keys/values are the latent queries/latents (softmax over the latents)
// (App. A.1, Table 2 in A.7).  FLARE++ first synthesises per-input queries
// with one more encode call and blends them onto fixed queries with a
// per-head gate (Sec. 3.2, App. A.4).
//
// Kernels (waves of 64; 32x32 MFMA tiles with the softmax axis on the
// accumulator column, so a lane's statistics are in-lane plus one
// permlane32 swap):
//   encode_dma_kernel -- bf16 split-N encode partials.  The flattened (head,
//                     token) range is cut into one contiguous piece per
//                     workgroup of 8 waves; 128-token K / V tiles arrive by
//                     LDS DMA one tile ahead, each wave owns 32 latents, and
//                     S^T = K Q^T and Z^T += V^T P^T run on MFMA.  A split
//                     emits (shift, sum, accumulator) and its keys' largest
//                     squared norm.
//   encode_kernel  -- the same for float32 inputs, register-staged tiles.
//   merge_kernel   -- log-sum-exp merge of the splits in a fixed order
//                     (Sec. 3.3, App. B.3); optionally the FLARE++ blend.
//   decode_kernel  -- per-token softmax over the latents: one 16-wave
//                     workgroup per compute unit keeps a head's scaled
//                     queries and latents in LDS, its waves claim 32-token
//                     blocks from an LDS counter, and S = Q K^T and
//                     Y^T += Z^T P run on MFMA with one lane per token column.
//   head_kernel    -- the whole FLARE or FLARE++ forward of one head in one
//                     16-wave workgroup (many short heads): the encode and
//                     decode code above with the split merges done in LDS.
//   latent_kernel  -- the FLARE++ encodes of one (head, latent block) per
//                     workgroup over all of the head's tokens, before the
//                     decode launch.
// proj.h holds the encode from the block input (K = X W_K, V = X W_V formed
// per tile), backward.h the reverse-mode kernels and their entry points,
// backward32.h the float32 ones.
// The bf16 paths bound the score error that the rounding of the pre-scaled
// queries can cause, per unit of work, and recompute exactly (queries split
// into bf16 hi + lo) where the bound exceeds kScoreErr.
// Scores are kept in log2 units: the queries are pre-multiplied by
// s*log2(e) so every exponential is a single v_exp_f32.  The bf16 loops use
// no shift at all (weights exp2(score), checked for range afterwards, with an
// exact-maximum recomputation as fallback) and sum the bf16 weights on the
// matrix core, so a score costs one exponential and half a pack on the VALU.
// float32 tiles keep an online softmax whose shift enters the score MFMA as
// its accumulator input and is only raised when a tile's maximum exceeds it
// by more than kTheta.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "flare.h"
#include "pieces.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;      // 4 waves per workgroup
constexpr int kTile = 128;         // tokens per float32 encode LDS tile (4 blocks of 32)
// Tokens per bf16 encode LDS tile (DMA-filled, double-buffered) for a
// workgroup of NW waves: 32 per wave up to 128, so two tiles of K and V stay
// within 64 KB and four waves per SIMD still fit.
template <int NW> constexpr int dma_rows() { return 128 < 32 * NW ? 128 : 32 * NW; }
constexpr int kDecWaves = 16;      // waves per decode workgroup: one workgroup per compute unit
constexpr int kDecThreads = 64 * kDecWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTheta = 8.0f;     // lazy-rescale threshold, log2 units
constexpr float kMinSum = 0x1p-64f;  // smallest weight sum the unshifted bf16 path accepts

// ----------------------------------------------------------------------------
// Small device helpers
// ----------------------------------------------------------------------------
template <typename T> __device__ inline float to_f(T x) { return (float)x; }
template <typename T> __device__ inline T from_f(float x) { return (T)x; }  // RNE for bf16
// fp16 values carried in bf16 registers and LDS (bit patterns), for score
// operands of normalised rows (see qk_mma_h)
__device__ inline bf16 h_bits(float x) { return __builtin_bit_cast(bf16, (_Float16)x); }
__device__ inline float h_val(bf16 b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (l % 32) and lane (l % 32) + 32, combined, on both lanes.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of the 32x32 MFMA accumulator held by register r of a lane in half g
// (the column is lane % 32): rows come in chunks of 4 consecutive rows.
__device__ inline int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ----------------------------------------------------------------------------
// MFMA operands.  A 32x32 product contracts over the feature axis d (QK) or
// over the 32 rows of a score tile (PV).
//   QK operand (one row: a token key or a latent query):
//     bf16: D/16 steps of 8 values, step st / half g / slot s <-> d = 16 st + 8 g + s
//     f32 : D/2 steps of 1 value,   step j  / half g          <-> d = g D/2 + j
//   PV A operand (one feature row d of a transposed value tile, 32 columns):
//     16 values at columns acc_row(j, g), j = 0..15, i.e. four runs of four.
// ----------------------------------------------------------------------------
template <typename T, int D> struct QKOp;
template <int D> struct QKOp<bf16, D> { bf16x8 v[D / 16]; };
template <int D> struct QKOp<float, D> { float v[D / 2]; };

template <typename T> struct PVOp;
template <> struct PVOp<bf16> { bf16x8 a0, a1; };
template <> struct PVOp<float> { float a[16]; };

template <int D> __device__ inline void zero_op(QKOp<bf16, D>& o) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int s = 0; s < 8; ++s) o.v[st][s] = (bf16)0.f;
}
template <int D> __device__ inline void zero_op(QKOp<float, D>& o) {
#pragma unroll
  for (int j = 0; j < D / 2; ++j) o.v[j] = 0.f;
}

// QK operand from a row already in the compute type (LDS or global).
template <int D> __device__ inline void load_op(QKOp<bf16, D>& o, const bf16* row, int g) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st) o.v[st] = *reinterpret_cast<const bf16x8*>(row + 16 * st + 8 * g);
}
template <int D> __device__ inline void load_op(QKOp<float, D>& o, const float* row, int g) {
#pragma unroll
  for (int j = 0; j < D / 2; j += 4) {
    f32x4 t = *reinterpret_cast<const f32x4*>(row + g * (D / 2) + j);
    o.v[j] = t[0]; o.v[j + 1] = t[1]; o.v[j + 2] = t[2]; o.v[j + 3] = t[3];
  }
}
// QK operand from a query row of type QT, multiplied by `scale` and rounded.
template <int D, typename QT> __device__ inline void load_op_scaled(QKOp<bf16, D>& o, const QT* row, int g, float scale) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int s = 0; s < 8; ++s) o.v[st][s] = (bf16)(to_f(row[16 * st + 8 * g + s]) * scale);
}
template <int D, typename QT> __device__ inline void load_op_scaled(QKOp<float, D>& o, const QT* row, int g, float scale) {
#pragma unroll
  for (int j = 0; j < D / 2; ++j) o.v[j] = to_f(row[g * (D / 2) + j]) * scale;
}

// ----------------------------------------------------------------------------
// Per-head RMS normalisation over the head dimension (FLARE++ paper, App. A.3
// and A.4, Table 2): N_0(x) = x / sqrt(mean_d x_d^2 + eps).  N_a adds a
// per-channel scale; the kernels move that scale onto the operand it
// multiplies (the queries, or the merged latents) and only ever apply N_0.
// ----------------------------------------------------------------------------
__device__ inline float norm_factor(float sumsq, int D, float eps) { return rsqrtf(sumsq / (float)D + eps); }

// QK operand (bf16) from a query row of type QT: optionally N_0 over the
// whole row (its other half is held by lane +-32, so all 64 lanes must call
// this), then multiplied channel by channel by the [D] rows mul0 and mul1
// (either may be null) and by `scale`, and rounded to bf16.  With lo given,
// lo receives the bf16 rounding of what that rounding left, so hi + lo is
// the scaled row to about 2^-17 of each element.  Returns the squared
// Euclidean norm of the rounding error of the whole row, |bf16(v) - v|^2.
// With H the row is rounded to fp16 instead (bit patterns; no lo), and an
// element beyond the fp16 range makes that error infinite.
template <int D, typename QT, bool H = false>
__device__ inline float load_q_row(QKOp<bf16, D>& o, QKOp<bf16, D>* lo, const QT* row, int g, float scale, bool norm,
                                   float eps, const float* mul0, const float* mul1, float* norm2 = nullptr) {
  float x[D / 2];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int s = 0; s < 8; ++s) x[8 * st + s] = to_f(row[16 * st + 8 * g + s]);
  float f = scale;
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < D / 2; ++j) ss += x[j] * x[j];
    f *= norm_factor(pair_sum(ss), D, eps);
  }
  float v[D / 2];  // x * f, then times the channel scales of this lane's features
#pragma unroll
  for (int j = 0; j < D / 2; ++j) v[j] = x[j] * f;
  if (mul0) {
#pragma unroll
    for (int j = 0; j < D / 2; ++j) v[j] *= mul0[16 * (j >> 3) + 8 * g + (j & 7)];
  }
  if (mul1) {
#pragma unroll
    for (int j = 0; j < D / 2; ++j) v[j] *= mul1[16 * (j >> 3) + 8 * g + (j & 7)];
  }
  float e2 = 0.f, n2 = 0.f;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float vs = v[8 * st + s];
      const bf16 h = H ? h_bits(vs) : (bf16)vs;
      const float r = vs - (H ? h_val(h) : (float)h);
      o.v[st][s] = h;
      if (lo) lo->v[st][s] = (bf16)r;
      e2 += r * r;
      n2 += vs * vs;
    }
  if (norm2) *norm2 = pair_sum(n2);  // the squared norm of the scaled row (before rounding)
  return pair_sum(e2);
}

// Scores from queries rounded to bf16 (the fast loops) differ from the exact
// ones by (bf16(q) - q) . k, at most |bf16(q) - q| |k| in absolute value (log2
// units).  A unit of work whose largest query rounding error times largest
// key norm stays within kScoreErr keeps the fast loop's result: every
// exponent is then within 2^-5 of the exact one.  Otherwise the work is redone
// with exact scores (queries as bf16 hi + lo).  Squared, as compared.
constexpr float kScoreErr2 = 0x1p-10f;

// Largest value over the 64 lanes of a wave, on every lane: within rows of
// 16 lanes by DPP quad and mirror moves, then across rows by the permlane
// swaps (no LDS traffic).
__device__ inline float dpp_max(float x, int ctrl) {
  float y;
  switch (ctrl) {  // the DPP control must be a constant
    case 0: y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)); break;  // xor 1
    case 1: y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)); break;  // xor 2
    case 2: y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)); break;  // half mirror
    default: y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)); break;  // mirror
  }
  return fmaxf(x, y);
}
__device__ inline float wave_max(float x) {
  x = dpp_max(dpp_max(dpp_max(dpp_max(x, 0), 1), 2), 3);  // the row's maximum on all 16 lanes
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));  // rows 2k and 2k + 1
  return pair_max(x);                                       // and the other half of the wave
}

// Squared Euclidean norm of a bf16 QK operand row (half in this lane, half in
// lane +-32; all 64 lanes must call this).
template <int D, bool H = false> __device__ inline float row_norm2(const QKOp<bf16, D>& o) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
  if constexpr (H) {  // fp16 elements
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int p = 0; p < 8; ++p) s += h_val(o.v[st][p]) * h_val(o.v[st][p]);
    return pair_sum(s);
  }
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bf16x2 v = {o.v[st][2 * p], o.v[st][2 * p + 1]};
      s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
    }
  return pair_sum(s);
}

// N_0 of a bf16 QK operand in registers (a key row, half in this lane and
// half in lane +-32; all 64 lanes must call this), rounded to bf16, or with H
// to fp16 bit patterns.  Returns the row's factor.
template <int D, bool H = false> __device__ inline float norm_op(QKOp<bf16, D>& o, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float v = (float)o.v[st][s];
      ss += v * v;
    }
  const float r = norm_factor(pair_sum(ss), D, eps);
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int s = 0; s < 8; ++s) o.v[st][s] = H ? h_bits((float)o.v[st][s] * r) : (bf16)((float)o.v[st][s] * r);
  return r;
}

template <int D> __device__ inline f32x16 qk_mma(const QKOp<bf16, D>& a, const QKOp<bf16, D>& b, f32x16 c) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v[st], b.v[st], c, 0, 0, 0);
  return c;
}
// Score operands of rows N_0-normalised on the fly: their elements are at
// most sqrt(D) in magnitude, so they are held as fp16 (bit patterns in the
// bf16 operand registers), whose 2^-11 rounding is 8 times finer than bf16's;
// the queries they meet are rounded to fp16 too.  The matrix core takes both
// formats at the same rate.
template <int D> __device__ inline f32x16 qk_mma_h(const QKOp<bf16, D>& a, const QKOp<bf16, D>& b, f32x16 c) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.v[st]), __builtin_bit_cast(f16x8, b.v[st]),
                                               c, 0, 0, 0);
  return c;
}
// the bf16 product, or with H the fp16 one
template <bool H, int D> __device__ inline f32x16 qk_mma_sel(const QKOp<bf16, D>& a, const QKOp<bf16, D>& b, f32x16 c) {
  if constexpr (H) return qk_mma_h<D>(a, b, c);
  else return qk_mma<D>(a, b, c);
}
template <int D> __device__ inline f32x16 qk_mma(const QKOp<float, D>& a, const QKOp<float, D>& b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < D / 2; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// PV A operand from row `xt` (a transposed tile row) starting at column base.
__device__ inline void load_pv(PVOp<bf16>& o, const bf16* xt, int g) {
  bf16x4 c0 = *reinterpret_cast<const bf16x4*>(xt + 4 * g);
  bf16x4 c1 = *reinterpret_cast<const bf16x4*>(xt + 8 + 4 * g);
  bf16x4 c2 = *reinterpret_cast<const bf16x4*>(xt + 16 + 4 * g);
  bf16x4 c3 = *reinterpret_cast<const bf16x4*>(xt + 24 + 4 * g);
  o.a0 = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
  o.a1 = __builtin_shufflevector(c2, c3, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline void load_pv(PVOp<float>& o, const float* xt, int g) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f32x4 t = *reinterpret_cast<const f32x4*>(xt + 8 * c + 4 * g);
    o.a[4 * c] = t[0]; o.a[4 * c + 1] = t[1]; o.a[4 * c + 2] = t[2]; o.a[4 * c + 3] = t[3];
  }
}
__device__ inline void zero_pv(PVOp<bf16>& o) {
#pragma unroll
  for (int s = 0; s < 8; ++s) { o.a0[s] = (bf16)0.f; o.a1[s] = (bf16)0.f; }
}
__device__ inline void zero_pv(PVOp<float>& o) {
#pragma unroll
  for (int j = 0; j < 16; ++j) o.a[j] = 0.f;
}

// acc += X^T P for float32 tiles, P being the exponentiated score tile in
// registers, plus the softmax denominator of this lane's column.  With D = 16
// the A operand's row 16 is all ones (see ones_pv), so accumulator row 16
// collects the column sums inside the MFMA; with D = 32 the weights are added.
template <int D> __device__ inline f32x16 pv_accum(const PVOp<float>& a, const f32x16& p, f32x16 acc, float& lsum) {
  if constexpr (D == 32) {
    float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 4) { t0 += p[j]; t1 += p[j + 1]; t2 += p[j + 2]; t3 += p[j + 3]; }
    lsum += (t0 + t1) + (t2 + t3);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[j], p[j], acc, 0, 0, 0);
  return acc;
}

// acc += X^T P for bf16 tiles from the packed weights (rows acc_row(0..7) in
// b0, acc_row(8..15) in b1).
__device__ inline f32x16 pv_mma(const PVOp<bf16>& a, const bf16x8& b0, const bf16x8& b1, f32x16 acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a0, b0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a1, b1, acc, 0, 0, 0);
  return acc;
}

// Softmax denominator of this lane's column, on both lanes of the pair.
template <typename T, int D> __device__ inline float col_sum(float lsum, const f32x16& acc) {
  if constexpr (sizeof(T) == 4 && D == 16) {  // accumulator row 16 = register 8 of the lower half
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[8]), __float_as_uint(acc[8]), false, false);
    return __uint_as_float(r[0]);
  } else {
    return pair_sum(lsum);
  }
}

// PV A operand of a lane whose feature row is beyond D: zero, except row 16
// (lanes 16 and 48), which is all ones when D = 16.
__device__ inline void ones_pv(PVOp<bf16>& o, int li, int D) {
  (void)li; (void)D;  // bf16 tiles get zero rows here (the forward's fast loops use pad_pv)
  const bf16 v = (bf16)0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) { o.a0[s] = v; o.a1[s] = v; }
}
__device__ inline void ones_pv(PVOp<float>& o, int li, int D) {
  const float v = D == 16 && li == 16 ? 1.f : 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) o.a[j] = v;
}
// The same for the unshifted bf16 loops of the forward: with D = 16 and
// matrix-core sums, row 16 is all ones, so accumulator row 16 (register 8 of
// the lower half) collects the column sums of the bf16 weights.
__device__ inline void pad_pv(PVOp<bf16>& o, int li, int D) {
  const bf16 v = (bf16)(D == 16 && li == 16 ? 1.f : 0.f);
#pragma unroll
  for (int s = 0; s < 8; ++s) { o.a0[s] = v; o.a1[s] = v; }
}

// Maximum of the tile column held by this lane pair.
__device__ inline float col_max(const f32x16& s) {
  float t = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) t = fmaxf(fmaxf(t, s[r]), s[r + 1]);
  return pair_max(fmaxf(t, s[15]));
}

// Raise the running shift of this lane's column by t: s, the shift (entered
// through the MFMA accumulator as -shift), the accumulator and the running
// sum follow.  The first non-empty tile sets the shift (nothing to rescale).
__device__ inline void raise_shift(float t, f32x16& s, f32x16& negshift, bool& started, float& lsum, f32x16& acc) {
  const float f = started ? fast_exp2(-t) : 0.f;
  s = s - t;
  negshift = negshift - t;
  acc = acc * f;
  lsum *= f;
  started = true;
}

// float32 tiles: one online-softmax step with the exact tile maximum.  On
// entry s = raw score - shift; on exit s holds the weights exp2(s).  The shift
// is raised to the tile maximum when that exceeds it by more than kTheta, or
// on the first non-empty tile.
__device__ inline void online_step(f32x16& s, f32x16& negshift, bool& started, float& lsum, f32x16& acc) {
  const float t = col_max(s);
  if ((t > kTheta) || (!started && t > -INFINITY)) raise_shift(t, s, negshift, started, lsum, acc);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r]);
}

// Weights already exponentiated, packed to bf16 (rows acc_row(0..7) in b0,
// acc_row(8..15) in b1).  Returns this lane's partial sum of the float32
// weights (plain adds: unlike packed dot products they issue alongside the
// MFMAs of other waves).
__device__ inline float pack_exps(const f32x16& p, bf16x8& b0, bf16x8& b1) {
#pragma unroll
  for (int r = 0; r < 8; ++r) { b0[r] = (bf16)p[r]; b1[r] = (bf16)p[8 + r]; }
  float t[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) t[r] = p[2 * r] + p[2 * r + 1];
  return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// Unshifted weights exp2(s) packed to bf16, without their sum.
__device__ inline void pack_only(const f32x16& s, bf16x8& b0, bf16x8& b1) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    b0[r] = (bf16)fast_exp2(s[r]);
    b1[r] = (bf16)fast_exp2(s[8 + r]);
  }
}

// Column sums of packed weight tiles on the matrix core.  A 16x16x32 product
// whose B operand is the packed tile (b0 or b1) of every lane sees lane l as
// column l % 16 and contraction group l / 16; lane l of the tile holds column
// l % 32 of the 32x32 weight tile.  The A operand below is all ones on lanes
// 0 and 32 (row 0, groups 0 and 2) and on lanes 17 and 49 (row 1, groups 1
// and 3), zero elsewhere, so row 0 of the 16x16 result sums tile columns
// 0..15 and row 1 tile columns 16..31, over both halves of the column.  The
// pairing holds for any order of the contraction inside a group, because A
// and B share it.  The sums are those of the bf16 weights the value product
// uses, so the normalised weights sum to one exactly as multiplied.
__device__ inline bf16x8 sum_selector(int lane) {
  const bf16 v = (bf16)((lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 1.f : 0.f);
  bf16x8 o;
#pragma unroll
  for (int s = 0; s < 8; ++s) o[s] = v;
  return o;
}
__device__ inline f32x4 sum_mma(const bf16x8& sel, const bf16x8& b0, const bf16x8& b1, f32x4 s) {
  s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, b0, s, 0, 0, 0);
  s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, b1, s, 0, 0, 0);
  return s;
}
// Sum of tile column li (on both lanes of the pair): row 0 / row 1 of the
// 16x16 result, column li % 16, held by lane li % 16 in registers 0 / 1.
__device__ inline float sum_col(const f32x4& s, int li) {
  const float a = __shfl(s[0], li & 15), b = __shfl(s[1], li & 15);
  return li < 16 ? a : b;
}

// Set rows at or beyond `from` (tile row index, acc_row order) to -inf.
__device__ inline void mask_rows(f32x16& s, int from, int g) {
  const int lim = from - 4 * g;  // acc_row(r, g) >= from  <=>  acc_row(r, 0) >= lim
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -INFINITY;
}

// One online-softmax step of the exact recomputations with the running shift
// held as one float per lane (the shift of this lane's column): on entry s is
// the raw score tile, on exit the weights exp2(s - shift).  The shift is
// raised to the tile maximum when that exceeds it by more than kTheta, or on
// the first non-empty tile; acc and lsum are rescaled with it.
__device__ inline void online_step_s(f32x16& s, float& shift, bool& started, float& lsum, f32x16& acc) {
  const float t = col_max(s);
  if ((t > shift + kTheta) || (!started && t > -INFINITY)) {
    const float f = started ? fast_exp2(shift - t) : 0.f;
    acc = acc * f;
    lsum *= f;
    shift = t;
    started = true;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r] - shift);
}

// bf16 fast path.  Softmax is invariant to the shift, and floating point is
// scale-invariant inside its exponent range, so the weights are taken as
// exp2(score) with no shift at all: the score MFMA starts from an inline
// zero, no maximum is tracked and every block is accumulated
// unconditionally.  The result equals the shifted computation up to rounding
// order as long as nothing leaves the range: a weight, running sum or
// accumulator that overflows becomes Inf and stays non-finite, and a column
// whose scores all lie far below zero shows a vanishing sum.  A sum of n
// weights that reaches kMinSum has a largest weight of at least kMinSum / n,
// so the weights lost to underflow (below 2^-126) are under 2^-62 n of it,
// far below bf16 resolution for any n < 2^40.  A column sum below kMinSum or
// a non-finite sum or accumulator sends that wave's work to a careful
// recomputation with the exact maximum of every block.  A sum can be NaN
// here even for finite inputs (an Inf weight times a zero selector in the
// matrix-core sums), so the test works on the exponent bits of a value the
// compiler cannot trace back to a float: built without NaN semantics, it
// would otherwise fold the test into an infinity check.
__device__ inline bool nonfinite(float x) {
  unsigned u = __float_as_uint(x);
  asm volatile("" : "+v"(u));
  return (u & 0x7f800000u) == 0x7f800000u;
}

// Column sum usable: finite and not vanishing.
__device__ inline bool fast_ok(float den) { return !nonfinite(den) && den >= kMinSum; }

// Encode partial usable: the column has no tokens (an empty split) or its sum
// passes fast_ok, and the accumulator is finite.
__device__ inline bool fast_failed(float den, bool has_tokens, const f32x16& acc) {
  bool bad = nonfinite(den) || (has_tokens && den < kMinSum);
#pragma unroll
  for (int r = 0; r < 16; ++r) bad = bad || nonfinite(acc[r]);
  return __builtin_amdgcn_ballot_w64(bad) != 0;
}

// ----------------------------------------------------------------------------
// bf16 tiles in LDS, row-major with 16-byte chunks XOR-swizzled per row so that
// 16 consecutive rows read at one chunk column, and 4 rows read across all
// chunks, hit distinct banks.  Tiles are filled by LDS DMA (global_load_lds,
// 16 bytes per lane, no VGPR staging); the PV operand gathers token columns
// with the transposing read ds_read_b64_tr_b16.
// ----------------------------------------------------------------------------
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D> __device__ inline int chunk_pos(int n, int c) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int sw = CPR == 4 ? ((n >> 2) & 3) : ((n >> 3) & 1);
  return n * CPR + (c ^ sw);
}

// Element offset of (row n, feature d) in a swizzled tile.
template <int D> __device__ inline int tile_off(int n, int d) { return chunk_pos<D>(n, d >> 3) * 8 + (d & 7); }

// Issue the DMA of rows [t0, t0 + dma_rows<NW>()) of a [*, D] bf16 matrix into a
// swizzled tile.  Rows at or beyond n_hi repeat row n_hi - 1 (they are masked
// out of the softmax by the caller), so no read leaves the matrix.
template <int D, int NW, int ROWS = dma_rows<NW>()>
__device__ inline void dma_tile(bf16* tile, const bf16* src, int t0, int n_hi, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int INSTR = ROWS * CPR / 64;  // 64 chunks (1 KB) per wave instruction
#pragma unroll
  for (int i = wave; i < INSTR; i += NW) {
    const int P = i * 64 + lane;
    const int n = P / CPR;
    const int c = (P % CPR) ^ (CPR == 4 ? ((n >> 2) & 3) : ((n >> 3) & 1));
    int row = t0 + n;
    row = row < n_hi ? row : n_hi - 1;
    __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)row * D + c * 8), (lds_void*)(tile + i * 512),
                                     16, 0, 0);
  }
}

__device__ inline void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// N_0 of every row of a swizzled bf16 tile in LDS, in place, once the tile's
// DMA is complete and visible to the workgroup.  Each thread takes one
// 16-byte chunk per pass; the D / 8 chunks of a row sit in consecutive lanes
// and add their partial sums with xor shuffles.  Rows past the piece repeat a
// valid row, so every row holds finite values.  With H the rows are written as
// fp16 (bit patterns; see qk_mma_h).
template <int D, int NW, int ROWS = dma_rows<NW>(), bool H = false>
__device__ inline void norm_tile(bf16* tile, int wave, int lane, float eps) {
  constexpr int CPR = D / 8;
  constexpr int CH = ROWS * CPR;
#pragma unroll
  for (int P0 = 0; P0 < CH; P0 += NW * 64) {
    const int P = P0 + wave * 64 + lane;
    if (P0 + wave * 64 < CH) {  // whole waves; CH is a multiple of 64
      bf16x8* ptr = reinterpret_cast<bf16x8*>(tile) + chunk_pos<D>(P / CPR, P % CPR);
      bf16x8 v = *ptr;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += (float)v[i] * (float)v[i];
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o);
      const float r = norm_factor(ss, D, eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = H ? h_bits((float)v[i] * r) : (bf16)((float)v[i] * r);
      *ptr = v;
    }
  }
}

// Running maximum of the squared key norms of a swizzled bf16 tile in LDS,
// once its DMA (and normalisation) is complete and visible: the NW waves
// split the tile's 16-byte chunks, and the D / 8 chunks of a row, held by
// consecutive lanes, add their partial sums by quad permutes.  Rows past the
// piece repeat its last row, so they add no key from outside it.
// With dst given, the tile's rows below nvalid are also copied to dst (row
// n at dst + n D, 16-byte chunks, coalesced).  H: the tile holds fp16 rows.
template <int D, int NW, int ROWS = dma_rows<NW>(), bool H = false>
__device__ inline float tile_key_max(const bf16* tile, int wave, int lane, float m, bf16* dst = nullptr,
                                     int nvalid = 0) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int CPR = D / 8;
  constexpr int CH = ROWS * CPR;  // a multiple of 64
  for (int P0 = wave * 64; P0 < CH; P0 += NW * 64) {
    const int P = P0 + lane;
    const bf16x8 v = reinterpret_cast<const bf16x8*>(tile)[chunk_pos<D>(P / CPR, P % CPR)];
    if (dst && P / CPR < nvalid) *reinterpret_cast<bf16x8*>(dst + (size_t)(P / CPR) * D + (P % CPR) * 8) = v;
    float s = 0.f;
    if constexpr (H) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s += h_val(v[i]) * h_val(v[i]);
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bf16x2 w = {v[2 * p], v[2 * p + 1]};
        s = __builtin_amdgcn_fdot2_f32_bf16(w, w, s, false);
      }
    }
    // lanes 4r .. 4r + 3 (D = 32) or 2r, 2r + 1 (D = 16) hold one row
    s += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0xB1, 0xF, 0xF, false));  // xor 1
    if constexpr (CPR == 4) s += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0x4E, 0xF, 0xF, false));
    m = fmaxf(m, s);
  }
  return m;
}

// Per-lane byte offsets into a swizzled tile for token block 0.  The XOR
// swizzle of a row only depends on the row index modulo 32, so token block nb
// adds nb * 64 * D bytes to every offset.
//   kq[st]: QK operand (key row li, chunk 2 st + g)
//   vq[k] : transposing read k of the PV operand: in a group of 16 lanes, lane
//           i points at row 8 k + 4 g + i/4, features d0 + 4 (i % 4) .. +3, so
//           lane j of the group receives feature d0 + j of rows 8 k + 4 g .. +3
//           (the four runs of acc_row).  Feature groups beyond D read
//           features 0..15 and are replaced by ones_pv afterwards.
template <int D> struct TileOffs {
  unsigned kq[D / 16];
  unsigned vq[4];
};
template <int D> __device__ inline TileOffs<D> tile_offsets(int lane) {
  TileOffs<D> o;
  const int li = lane & 31, g = lane >> 5;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) o.kq[st] = chunk_pos<D>(li, 2 * st + g) * 16;
  const int i = lane & 15, q = lane >> 4;
  const int d0 = 16 * (q & 1);
  const int d = (d0 < D ? d0 : 0) + 4 * (i & 3);
#pragma unroll
  for (int k = 0; k < 4; ++k) o.vq[k] = tile_off<D>(8 * k + 4 * g + (i >> 2), d) * 2;
  return o;
}

__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <typename V> __device__ inline V lds_load(unsigned addr) {
  return *(const __attribute__((address_space(3))) V*)(uintptr_t)addr;
}

// The transposing reads are issued as inline assembly: the compiler does not
// know which LDS bytes the builtin touches and would otherwise wait for every
// DMA in flight (including the one filling the other buffer) before each
// read.  pv_wait() must run before the operand is used; it takes the operand
// as an in/out value so no use can be scheduled ahead of it.  Only tiles whose
// DMA completed before the last barrier are read this way.
template <int OFF> __device__ inline bf16x4 tr_read(unsigned addr) {
  bf16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
__device__ inline void pv_wait(PVOp<bf16>& o, int lane, int D) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(o.a0), "+v"(o.a1));
  if (16 * ((lane >> 4) & 1) >= D) ones_pv(o, lane & 31, D);  // feature rows beyond D
}
// The forward encode's: feature rows beyond D padded by pad_pv.
__device__ inline void pv_wait_pad(PVOp<bf16>& o, int lane, int D) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(o.a0), "+v"(o.a1));
  if (16 * ((lane >> 4) & 1) >= D) pad_pv(o, lane & 31, D);
}

// ----------------------------------------------------------------------------
// Encode partials
// ----------------------------------------------------------------------------
struct EncArgs {
  const void* Q;      // [H,M,D] or [B,H,M,D], type QT
  const void* K;      // [B,H,N,D], type T
  const void* V;      // [B,H,N,D], type T (may equal K)
  float* part_acc;    // [nbh][pmax][M][D]
  float2* part_al;    // [nbh][pmax][M]   (shift in log2 units, sum)
  float* part_km;     // [nbh][pmax] largest squared key norm of each split's keys, or null (bf16)
  long long total;    // nbh * N
  int q_batched, v_alias, H, N, M, G, nwg, pmax, bh0;
  int m0 = 0;         // first latent of the workgroup's G latent blocks (bf16 encode)
  float qscale;       // s * log2(e)
  // query rows: N_0 when norm_q, then channel scales qmul0 / qmul1 ([H, D] or
  // null); keys N_0 per row when the kernel's NK flag is set (bf16 only)
  int norm_q;
  const float* qmul0;
  const float* qmul1;
  float eps;
};

template <typename T, int D> struct EncLds {
  static constexpr int E = 16 / sizeof(T);             // elements per 16 bytes
  static constexpr int KST = D + E;                    // K row stride
  static constexpr int VST = kTile + (sizeof(T) == 2 ? 8 : 4);  // V^T row stride
  static constexpr int BUF = kTile * KST + D * VST;    // elements per buffer
  static constexpr bool DB = sizeof(T) == 2;           // double-buffered tiles
  static constexpr int VPT = kTile * D / E / kThreads; // 16-byte vectors per thread per tensor
  static constexpr size_t bytes = (size_t)BUF * sizeof(T) * (DB ? 2 : 1);
};

template <typename T, int D>
__device__ inline void enc_fetch(uint4* kr, uint4* vr, const T* Kh, const T* Vh, bool v_alias, int t0, int n_hi) {
  using L = EncLds<T, D>;
  constexpr int RV = D / L::E;  // vectors per row
#pragma unroll
  for (int i = 0; i < L::VPT; ++i) {
    const int v = threadIdx.x + kThreads * i;
    const int n = v / RV, c = (v % RV) * L::E;
    const int row = t0 + n;
    if (row < n_hi) {
      kr[i] = *reinterpret_cast<const uint4*>(Kh + (size_t)row * D + c);
      vr[i] = v_alias ? kr[i] : *reinterpret_cast<const uint4*>(Vh + (size_t)row * D + c);
    } else {
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <typename T, int D>
__device__ inline void enc_stash(T* buf, const uint4* kr, const uint4* vr) {
  using L = EncLds<T, D>;
  constexpr int RV = D / L::E;
  T* ks = buf;
  T* vt = buf + kTile * L::KST;
#pragma unroll
  for (int i = 0; i < L::VPT; ++i) {
    const int v = threadIdx.x + kThreads * i;
    const int n = v / RV, c = (v % RV) * L::E;
    *reinterpret_cast<uint4*>(ks + n * L::KST + c) = kr[i];
    const T* e = reinterpret_cast<const T*>(&vr[i]);
#pragma unroll
    for (int j = 0; j < L::E; ++j) vt[(c + j) * L::VST + n] = e[j];
  }
}

template <typename T, typename QT, int D, int MBW>
__global__ void __launch_bounds__(kThreads) encode_kernel(EncArgs a) {
  using L = EncLds<T, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);
  // the wave index is uniform: kept in a scalar register, block guards derived
  // from it become scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int G = a.G, WN = 4 / G;
  const int mg = wave % G, ng = wave / G;
  const int N = a.N, M = a.M;

  long long x = piece_start(blockIdx.x, a.total, a.nwg);
  const long long xe = piece_start(blockIdx.x + 1, a.total, a.nwg);
  while (x < xe) {
    const int bhl = (int)(x / N);
    const long long hb = (long long)bhl * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int bh = a.bh0 + bhl;
    const int h = bh % a.H, b = bh / a.H;
    const int slot = (blockIdx.x - piece_of(hb, a.total, a.nwg)) * WN + ng;

    // This wave's latent queries (B operand: column = latent), scaled to log2 units.
    const QT* Qh = reinterpret_cast<const QT*>(a.Q) + (size_t)(a.q_batched ? bh : h) * M * D;
    QKOp<T, D> qop[MBW];
    f32x16 negs[MBW], acc[MBW];
    float lsum[MBW];
    bool started[MBW];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int m = (mg * MBW + mb) * 32 + li;
      if (m < M) load_op_scaled<D>(qop[mb], Qh + (size_t)m * D, g, a.qscale);
      else zero_op<D>(qop[mb]);
#pragma unroll
      for (int r = 0; r < 16; ++r) { negs[mb][r] = 0.f; acc[mb][r] = 0.f; }
      lsum[mb] = 0.f;
      started[mb] = false;
    }
    (void)b;

    const T* Kh = reinterpret_cast<const T*>(a.K) + (size_t)bh * N * D;
    const T* Vh = reinterpret_cast<const T*>(a.V) + (size_t)bh * N * D;
    uint4 kr[L::VPT], vr[L::VPT];
    enc_fetch<T, D>(kr, vr, Kh, Vh, a.v_alias, n_lo, n_hi);
    __syncthreads();  // the previous piece is done with buffer 0
    enc_stash<T, D>(lds, kr, vr);
    __syncthreads();
    int buf = 0;
    for (int t0 = n_lo; t0 < n_hi; t0 += kTile) {
      const bool more = t0 + kTile < n_hi;
      if (more) enc_fetch<T, D>(kr, vr, Kh, Vh, a.v_alias, t0 + kTile, n_hi);
      const T* ks = lds + buf * L::BUF;
      const T* vt = ks + kTile * L::KST;
      for (int nb = ng; nb < kTile / 32; nb += WN) {
        const int row0 = t0 + 32 * nb;
        if (row0 >= n_hi) break;
        QKOp<T, D> kop;
        load_op<D>(kop, ks + (32 * nb + li) * L::KST, g);
        PVOp<T> vop;
        if (li < D) load_pv(vop, vt + li * L::VST + 32 * nb, g);
        else ones_pv(vop, li, D);
        const bool tail = row0 + 32 > n_hi;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
          f32x16 s = qk_mma<D>(kop, qop[mb], negs[mb]);
          if (tail) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (row0 + acc_row(r, g) >= n_hi) s[r] = -INFINITY;
          }
          online_step(s, negs[mb], started[mb], lsum[mb], acc[mb]);
          acc[mb] = pv_accum<D>(vop, s, acc[mb], lsum[mb]);
        }
      }
      if (L::DB) {
        if (more) enc_stash<T, D>(lds + (buf ^ 1) * L::BUF, kr, vr);
        __syncthreads();
        buf ^= 1;
      } else {
        __syncthreads();
        if (more) enc_stash<T, D>(lds, kr, vr);
        __syncthreads();
      }
    }

    // Emit this wave's split: per latent (shift, sum) and the accumulator.
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int m = (mg * MBW + mb) * 32 + li;
      const float ltot = col_sum<float, D>(lsum[mb], acc[mb]);
      if (m < M) {
        const size_t p = (size_t)bhl * a.pmax + slot;
        float* dst = a.part_acc + (p * M + m) * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (8 * c + 4 * g < D) {
            f32x4 v = {acc[mb][4 * c], acc[mb][4 * c + 1], acc[mb][4 * c + 2], acc[mb][4 * c + 3]};
            *reinterpret_cast<f32x4*>(dst + 8 * c + 4 * g) = v;
          }
        }
        if (g == 0) a.part_al[p * M + m] = make_float2(-negs[mb][0], ltot);
      }
    }
    x = hb + n_hi;
  }
}

// Running weight sum of the unshifted bf16 loops: the 16x16 matrix-core sums
// and their selector operand, or a lane's partial sum of float32 weights.
template <bool MMA, int D> struct WSum;
template <> struct WSum<true, 32> {  // 16x16x32 sums of the packed weights
  f32x4 s;
  bf16x8 sel;
  __device__ explicit WSum(int lane) : s{0.f, 0.f, 0.f, 0.f}, sel(sum_selector(lane)) {}
  __device__ void add(const f32x16& sc, bf16x8& b0, bf16x8& b1) {
    pack_only(sc, b0, b1);
    s = sum_mma(sel, b0, b1, s);
  }
  __device__ float total(int li, const f32x16&) const { return sum_col(s, li); }
};
template <> struct WSum<true, 16> {  // accumulator row 16 (pad_pv)
  __device__ explicit WSum(int) {}
  __device__ void add(const f32x16& sc, bf16x8& b0, bf16x8& b1) { pack_only(sc, b0, b1); }
  __device__ float total(int, const f32x16& acc) const { return col_sum<float, 16>(0.f, acc); }
};
template <int D> using RowSum = WSum<true, D>;

// Scores S^T = K Q^T of token block NB of the tile in buffer BO (LDS byte
// addresses ka + BO + NB * 64 * D) against one wave's 32 latents, unshifted.
// The key reads are inline assembly, like the transposing reads: as ordinary
// loads the compiler cannot tell them from the DMA filling the other buffer
// and would make them wait for it.
template <int OFF> __device__ inline bf16x8 k_read(unsigned addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int D, int NB, int BO, bool H = false>
__device__ inline f32x16 enc_scores(const unsigned (&ka)[D / 16], const QKOp<bf16, D>& qop) {
  constexpr int OFF = BO + NB * 64 * D;
  QKOp<bf16, D> kop;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) kop.v[st] = k_read<OFF>(ka[st]);
  if constexpr (D == 32) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kop.v[0]), "+v"(kop.v[1]));
  else asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kop.v[0]));
  return qk_mma_sel<H, D>(kop, qop, f32x16{});
}

// Weights of those scores into the running sum and Z^T += V^T P^T.  row0 is
// the block's first token, n_hi the end of the piece: rows at or past n_hi
// (all of them for a block past the end) get no weight.
template <int D, int NB, int BO>
__device__ inline void enc_consume(const unsigned (&va)[4], f32x16 sc, int row0, int n_hi, int g, int lane,
                                   RowSum<D>& lsum, f32x16& acc) {
  constexpr int OFF = BO + NB * 64 * D;
  PVOp<bf16> vop;
  {
    const bf16x4 r0 = tr_read<OFF>(va[0]), r1 = tr_read<OFF>(va[1]);
    const bf16x4 r2 = tr_read<OFF>(va[2]), r3 = tr_read<OFF>(va[3]);
    vop.a0 = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    vop.a1 = __builtin_shufflevector(r2, r3, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  if (row0 + 32 > n_hi) mask_rows(sc, n_hi - row0, g);
  bf16x8 b0, b1;
  lsum.add(sc, b0, b1);
  pv_wait_pad(vop, lane, D);
  acc = pv_mma(vop, b0, b1, acc);
}

// Blocks J, J + 1, ... of one wave's share of a tile (block J is token block
// J WN of the tile, its scores already issued in `cur`).  The scores of the
// next block are issued before the current block's weights are
// exponentiated, so the MFMAs run under the exponentials.  Blocks past the
// end of the piece are computed and masked to zero weight (their rows repeat
// the piece's last row): a branch per block costs more than the rare waste.
// H: keys and queries are fp16 (see qk_mma_h).
template <int D, int WN, int BO, int J, int NBLK, bool H = false>
__device__ inline void encode_chain(const unsigned (&ka)[D / 16], const unsigned (&va)[4], int t0, int n_hi, int g,
                                    int lane, const QKOp<bf16, D>& qop, RowSum<D>& lsum, f32x16& acc, const f32x16& cur) {
  if constexpr (J + 1 < NBLK) {
    const f32x16 nxt = enc_scores<D, (J + 1) * WN, BO, H>(ka, qop);
    enc_consume<D, J * WN, BO>(va, cur, t0 + 32 * J * WN, n_hi, g, lane, lsum, acc);
    encode_chain<D, WN, BO, J + 1, NBLK, H>(ka, va, t0, n_hi, g, lane, qop, lsum, acc, nxt);
  } else {
    enc_consume<D, J * WN, BO>(va, cur, t0 + 32 * J * WN, n_hi, g, lane, lsum, acc);
  }
}

// The ROWS-token tile at t0 for one wave: token blocks ng, ng + WN, ... (the
// per-wave offset ng * 64 * D is already folded into ka / va, and t0 here is
// the wave's first row).
template <int D, int NW, int WN, int BO, int ROWS = dma_rows<NW>(), bool H = false>
__device__ inline void encode_tile(const unsigned (&ka)[D / 16], const unsigned (&va)[4], int t0, int n_hi, int g,
                                   int lane, const QKOp<bf16, D>& qop, RowSum<D>& lsum, f32x16& acc) {
  if (t0 >= n_hi) return;
  constexpr int NBLK = ROWS / 32 / WN;
  static_assert(NBLK >= 1, "a tile holds at least one token block per wave");
  encode_chain<D, WN, BO, 0, NBLK, H>(ka, va, t0, n_hi, g, lane, qop, lsum, acc, enc_scores<D, 0, BO, H>(ka, qop));
}

// Careful recomputation of one wave's share of a piece (the token blocks
// t0 + 32 (ng + k WN) of every `rows`-token tile), straight from global memory
// with exact scores (the scaled queries as bf16 hi + lo, two products) and
// the exact maximum of every block (online softmax with a shift raised
// whenever the block maximum exceeds it by more than kTheta).  Used only when
// the fast loop's rounded queries could shift a score by more than its bound,
// or its weights left the float range.
// With NK the key rows are N_0-normalised as they are loaded, and so are the
// values when they alias the keys.  Returns the final shift of this lane's
// latent.
template <int D, bool NK>
__device__ inline float encode_careful(const bf16* Kh, const bf16* Vh, bool alias, float eps, int n_lo, int n_hi,
                                       int ng, int WN, int rows, int lane, const QKOp<bf16, D>& qhi,
                                       const QKOp<bf16, D>& qlo, float& lsum, f32x16& acc) {
  const int li = lane & 31, g = lane >> 5;
  float shift = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  lsum = 0.f;
  bool started = false;
  for (int t0 = n_lo; t0 < n_hi; t0 += rows) {
    for (int nb = ng; nb < rows / 32; nb += WN) {
      const int row0 = t0 + 32 * nb;
      if (row0 >= n_hi) break;
      QKOp<bf16, D> kop;
      load_op<D>(kop, Kh + (size_t)(row0 + li < n_hi ? row0 + li : n_hi - 1) * D, g);
      float r = 1.f;  // N_0 factor of key row row0 + li
      if constexpr (NK) r = norm_op<D>(kop, eps);
      if (row0 + li >= n_hi) zero_op<D>(kop);
      PVOp<bf16> vop;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int n = row0 + acc_row(j, g);
        float v = (li < D && n < n_hi) ? (float)Vh[(size_t)n * D + li] : 0.f;
        if constexpr (NK) {
          const float rn = __shfl(r, acc_row(j, g));  // factor of row n, held by lane n - row0
          if (alias) v = (float)(bf16)(v * rn);       // the same rounding as the normalised tile
        }
        if (j < 8) vop.a0[j] = (bf16)v;
        else vop.a1[j - 8] = (bf16)v;
      }
      f32x16 sc = qk_mma<D>(kop, qlo, qk_mma<D>(kop, qhi, f32x16{}));
      if (row0 + 32 > n_hi) mask_rows(sc, n_hi - row0, g);
      online_step_s(sc, shift, started, lsum, acc);
      bf16x8 b0, b1;
      lsum += pack_exps(sc, b0, b1);
      acc = pv_mma(vop, b0, b1, acc);
    }
  }
  return shift;
}

// bf16 encode: NW waves in WN token lanes of G = NW / WN latent groups; wave w
// owns latent block w % G (32 latents) and token blocks w / G + k WN of every
// ROWS-token tile.  Tiles are double-buffered in two distinct LDS arrays: the
// DMA of the next tile is in flight while the current one is consumed.
// Piece `piece` of a.nwg (the workgroup's); tiles: 4 ROWS D bf16 of LDS
// ([buffer][K, V]), kred: NW floats of LDS (per-wave largest squared key norm
// of a piece).  The waves' latents start at a.m0.  With LP the workgroup's
// piece is one whole head and its split partials go to LDS, lacc
// [WN][32 G][D] and lal [WN][32 G] (split = token lane, latents from a.m0),
// and a.part_km, when set, receives the head's largest squared key norm at
// the head's index.
template <typename QT, int D, int NW, int WN, bool NK, int ROWS = dma_rows<NW>(), bool LP = false, bool H = false>
__device__ __attribute__((always_inline)) inline void encode_dma_body(const EncArgs& a, int piece, bf16* tiles,
                                                                      float* kred, float* lacc = nullptr,
                                                                      float2* lal = nullptr) {
  constexpr int TE = ROWS * D;  // elements per tile
  constexpr int G = NW / WN;
  bf16* const k0 = tiles;
  bf16* const v0 = tiles + TE;
  bf16* const k1 = tiles + 2 * TE;
  bf16* const v1 = tiles + 3 * TE;
  // the wave index is uniform: kept in a scalar register, block guards derived
  // from it become scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int mg = wave % G, ng = wave / G;
  const int N = a.N, M = a.M;
  const bool alias = a.v_alias;

  // LDS byte addresses of this lane's operands in buffer 0; buffer 1 is a
  // fixed distance further (folded into the read offsets)
  const TileOffs<D> to = tile_offsets<D>(lane);
  const unsigned wofs = ng * 64 * D;
  unsigned ka[D / 16], va[4];
  {
    const unsigned bk = lds_addr(k0) + wofs, bv = lds_addr(alias ? k0 : v0) + wofs;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) ka[st] = bk + to.kq[st];
#pragma unroll
    for (int k = 0; k < 4; ++k) va[k] = bv + to.vq[k];
  }

  long long x = piece_start(piece, a.total, a.nwg);
  const long long xe = piece_start(piece + 1, a.total, a.nwg);
  while (x < xe) {
    const int bhl = (int)(x / N);
    const long long hb = (long long)bhl * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int bh = a.bh0 + bhl;
    const int h = bh % a.H;
    const int slot = (piece - piece_of(hb, a.total, a.nwg)) * WN + ng;

    // this lane's latent query row (rows past M repeat row M - 1 and are zeroed)
    auto qrow = [&]() {
      const int m = a.m0 + mg * 32 + li;
      return reinterpret_cast<const QT*>(a.Q) + ((size_t)(a.q_batched ? bh : h) * M + (m < M ? m : M - 1)) * D;
    };
    const float* qm0 = a.qmul0 ? a.qmul0 + (size_t)h * D : nullptr;
    const float* qm1 = a.qmul1 ? a.qmul1 + (size_t)h * D : nullptr;
    const int m = a.m0 + mg * 32 + li;
    QKOp<bf16, D> qop;
    // the wave's largest query rounding error (uniform: a scalar register)
    const float qerr2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(
        wave_max(load_q_row<D, QT, H>(qop, nullptr, qrow(), g, a.qscale, a.norm_q != 0, a.eps, qm0, qm1)))));
    if (m >= M) zero_op<D>(qop);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    RowSum<D> wsum(lane);
    float kmax2 = 0.f;  // largest squared key norm of the tiles this wave scanned

    const bf16* Kh = reinterpret_cast<const bf16*>(a.K) + (size_t)bh * N * D;
    const bf16* Vh = reinterpret_cast<const bf16*>(a.V) + (size_t)bh * N * D;
    __syncthreads();  // the previous piece is done with the tiles
    dma_tile<D, NW, ROWS>(k0, Kh, n_lo, n_hi, wave, lane);
    if (!alias) dma_tile<D, NW, ROWS>(v0, Vh, n_lo, n_hi, wave, lane);
    wait_dma();
    __syncthreads();
    if constexpr (NK) {  // key rows N_0 in place (and the values with them when they alias)
      norm_tile<D, NW, ROWS, H>(k0, wave, lane, a.eps);
      __syncthreads();
    }
    for (int t0 = n_lo; t0 < n_hi; t0 += 2 * ROWS) {
      // tile t0 from buffer 0 while tile t0 + ROWS streams into buffer 1
      const int tn = t0 + ROWS;
      kmax2 = tile_key_max<D, NW, ROWS, H>(k0, wave, lane, kmax2);
      if (tn < n_hi) {
        dma_tile<D, NW, ROWS>(k1, Kh, tn, n_hi, wave, lane);
        if (!alias) dma_tile<D, NW, ROWS>(v1, Vh, tn, n_hi, wave, lane);
      }
      encode_tile<D, NW, WN, 0, ROWS, H>(ka, va, t0 + 32 * ng, n_hi, g, lane, qop, wsum, acc);
      wait_dma();
      __syncthreads();
      if (tn >= n_hi) break;
      if constexpr (NK) {
        norm_tile<D, NW, ROWS, H>(k1, wave, lane, a.eps);
        __syncthreads();
      }
      // tile tn from buffer 1 while tn + ROWS streams into buffer 0
      const int tn2 = tn + ROWS;
      kmax2 = tile_key_max<D, NW, ROWS, H>(k1, wave, lane, kmax2);
      if (tn2 < n_hi) {
        dma_tile<D, NW, ROWS>(k0, Kh, tn2, n_hi, wave, lane);
        if (!alias) dma_tile<D, NW, ROWS>(v0, Vh, tn2, n_hi, wave, lane);
      }
      if constexpr (2 * TE * 2 < 32768) {
        encode_tile<D, NW, WN, 2 * TE * 2, ROWS, H>(ka, va, tn + 32 * ng, n_hi, g, lane, qop, wsum, acc);
      } else {  // buffer 1 beyond the reads' 16-bit offsets: its addresses in registers
        unsigned kb[D / 16], vb[4];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) kb[st] = ka[st] + 2 * TE * 2;
#pragma unroll
        for (int k = 0; k < 4; ++k) vb[k] = va[k] + 2 * TE * 2;
        encode_tile<D, NW, WN, 0, ROWS, H>(kb, vb, tn + 32 * ng, n_hi, g, lane, qop, wsum, acc);
      }
      wait_dma();
      __syncthreads();
      if constexpr (NK) {
        if (tn2 < n_hi) {
          norm_tile<D, NW, ROWS, H>(k0, wave, lane, a.eps);
          __syncthreads();
        }
      }
    }
    // The piece's largest key norm (every wave scanned part of every tile).
    // kred is free: its last readers passed the barriers of this piece's tiles.
    kmax2 = wave_max(kmax2);
    if (lane == 0) kred[wave] = kmax2;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) kmax2 = fmaxf(kmax2, kred[w]);
    if constexpr (LP) {
      if (a.part_km && threadIdx.x == 0) a.part_km[bh] = kmax2;
    } else {
      if (a.part_km && threadIdx.x < WN)  // the same for each of the piece's WN splits
        a.part_km[(size_t)bhl * a.pmax + slot - ng + threadIdx.x] = kmax2;
    }
    // unshifted partial (see fast_ok), renormalised to a power-of-two shift
    // so that the merge never adds sums beyond the float range; or the exact
    // recomputation when the rounded queries could move a score too far.
    // Lane indices are taken again from an index opaque to the compiler, so
    // that none is held in a register across the tile loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane2 = tid & 63, li2 = lane2 & 31, g2 = lane2 >> 5, ml2 = mg * 32 + li2, m2 = a.m0 + ml2;
    float ltot = wsum.total(li2, acc), shift = 0.f;
    const bool inexact = qerr2 * kmax2 > kScoreErr2;
    if (inexact || fast_failed(ltot, n_lo + 32 * ng < n_hi, acc)) {
      const QT* qr = reinterpret_cast<const QT*>(a.Q) + ((size_t)(a.q_batched ? bh : h) * M + (m2 < M ? m2 : M - 1)) * D;
      QKOp<bf16, D> qhi, qlo;
      load_q_row<D>(qhi, &qlo, qr, g2, a.qscale, a.norm_q != 0, a.eps, qm0, qm1);
      if (m2 >= M) { zero_op<D>(qhi); zero_op<D>(qlo); }
      float lsum;
      shift = encode_careful<D, NK>(Kh, alias ? Kh : Vh, alias, a.eps, n_lo, n_hi, ng, WN, ROWS, lane2, qhi, qlo,
                                    lsum, acc);
      ltot = pair_sum(lsum);
    } else {
      const int e = __builtin_amdgcn_frexp_expf(ltot);  // ltot = f 2^e, f in [1/2, 1); 0 for an empty split
      const float sc = __builtin_amdgcn_ldexpf(1.f, -e);
      acc = acc * sc;
      ltot *= sc;
      shift = (float)e;
    }
    if (m2 < M) {
      // LP: [WN][32 G][D] over the workgroup's latents; else [pmax][M][D] per head
      const size_t p = LP ? (size_t)slot : (size_t)bhl * a.pmax + slot;
      const size_t row = LP ? p * (32 * G) + ml2 : p * M + m2;
      float* dst = (LP ? lacc : a.part_acc) + row * D;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (8 * c + 4 * g2 < D) {
          f32x4 v = {acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
          *reinterpret_cast<f32x4*>(dst + 8 * c + 4 * g2) = v;
        }
      }
      if (g2 == 0) (LP ? lal : a.part_al)[row] = make_float2(shift, ltot);
    }
    x = hb + n_hi;
  }
}

template <typename QT, int D, int NW, int WN, bool NK, bool H = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) encode_dma_kernel(EncArgs a) {
  __shared__ __align__(16) bf16 tiles[4 * dma_rows<NW>() * D];
  __shared__ float kred[NW];
  encode_dma_body<QT, D, NW, WN, NK, dma_rows<NW>(), false, H>(a, blockIdx.x, tiles, kred);
}

// ----------------------------------------------------------------------------
// Merge of the splits (Sec. 3.3 / App. B.3): with a_p the shift and l_p the sum
// of split p, A = max over non-empty splits of a_p, w_p = 2^(a_p - A):
//   Z = sum_p w_p U_p / sum_p w_p l_p,   L = ln2 (A + log2 sum_p w_p l_p).
// A split with no tokens has l_p = 0 and is skipped; if every split is empty
// Z = 0 and L = -inf (App. B.3).  Blend mode writes Qout = Qf + gate * Z.
// ----------------------------------------------------------------------------
struct MergeArgs {
  const float* part_acc;
  const float2* part_al;
  float* Z;           // [B,H,M,D] (global head index), or null in blend mode
  float* L;           // [B,H,M] or null
  const void* Qf;     // [H,M,D] of type QT, blend mode only
  const float* gate;  // [H]
  float* Qout;        // [B,H,M,D], blend mode only
  const float* part_km;  // the encode's per-split key-norm maxima, or null
  float* kmax;           // [B H] per head: their maximum (global head index), or null
  long long total;
  int N, M, D, H, WN, nwg, pmax, bh0, nbh;
  int norm_qf;        // blend with N_0(Qf) instead of Qf
  const float* zmul;  // [H, D] channel scale of Z (the values' N_a scale), or null
  float eps;
};

// Running (A, den, num) of a set of splits: max shift, and sum of l_p and of
// U_p scaled to 2^A.  Empty sets have A = -inf, den = num = 0.
struct MergeState {
  float A, den;
  f32x4 num;  // four features of the latent
};

__device__ inline MergeState merge_fold(MergeState s, float a, float l, const f32x4& u) {
  if (l > 0.f) {
    if (a > s.A) {
      const float f = fast_exp2(s.A - a);  // 0 while A = -inf
      s.den *= f;
      s.num = s.num * f;
      s.A = a;
    }
    const float w = fast_exp2(a - s.A);
    s.den += w * l;
    s.num += w * u;
  }
  return s;
}

__device__ inline MergeState merge_pair(MergeState x, MergeState y) {
  const float A = fmaxf(x.A, y.A);
  if (!(A > -INFINITY)) return x;
  const float fx = x.A > -INFINITY ? fast_exp2(x.A - A) : 0.f;
  const float fy = y.A > -INFINITY ? fast_exp2(y.A - A) : 0.f;
  return MergeState{A, x.den * fx + y.den * fy, x.num * fx + y.num * fy};
}

constexpr int kMergeBatch = 8;  // splits loaded per lane group before any is folded

// One wave per (head, latent).  Lane (pg, c) owns features 4c .. 4c + 3 and
// folds the splits p = pg, pg + PGW, ... (PGW = 64 / (D / 4) lane groups) in
// ascending order, all of a batch's loads issued before any is folded; the
// PGW group states are then combined by a fixed xor butterfly over the group
// bits of the lane, and group 0 writes the result.
template <typename QT>
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  // B H M < 2^31 (checked on the host): 32-bit index arithmetic
  const unsigned pair = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (pair >= (unsigned)a.nbh * (unsigned)a.M) return;  // the whole wave
  const int D = a.D, CPS = D / 4, PGW = 64 / CPS;
  const int pg = lane / CPS, c = lane % CPS;
  const int m = (int)(pair % (unsigned)a.M);
  const int bhl = (int)(pair / (unsigned)a.M);
  const int bh = a.bh0 + bhl;
  MergeState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (a.N == 0 && a.kmax && m == 0 && lane == 0) a.kmax[bh] = 0.f;
  if (a.N > 0) {
    const long long hb = (long long)bhl * a.N;
    const int cnt = (piece_of(hb + a.N - 1, a.total, a.nwg) - piece_of(hb, a.total, a.nwg) + 1) * a.WN;
    const size_t base = (size_t)bhl * a.pmax;
    if (a.kmax && m == 0) {  // the head's largest key norm, for the decode (every lane active)
      float km = 0.f;
      for (int p = lane; p < cnt; p += 64) km = fmaxf(km, a.part_km[base + p]);
      km = wave_max(km);
      if (lane == 0) a.kmax[bh] = km;
    }
    // slots past cnt load nothing and count as empty
    for (int p0 = pg; p0 < cnt; p0 += kMergeBatch * PGW) {
      float2 v[kMergeBatch];
      f32x4 u[kMergeBatch];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const int p = p0 + j * PGW;
        v[j] = make_float2(-INFINITY, 0.f);
        u[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p < cnt) {
          const size_t i = (base + p) * a.M + m;
          v[j] = a.part_al[i];
          u[j] = reinterpret_cast<const f32x4*>(a.part_acc + i * D)[c];
        }
      }
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) asm volatile("" ::"v"(v[j]), "v"(u[j]));
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) st = merge_fold(st, v[j].x, p0 + j * PGW < cnt ? v[j].y : 0.f, u[j]);
    }
  }
  for (int o = CPS; o < 64; o <<= 1) {
    MergeState t;
    t.A = __shfl_xor(st.A, o);
    t.den = __shfl_xor(st.den, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.num[i] = __shfl_xor(st.num[i], o);
    st = merge_pair(st, t);
  }
  const int h = bh % a.H;
  float qf[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.Qout) {  // blend mode: the fixed query, N_0 over its D features while every lane group is active
    const QT* q = reinterpret_cast<const QT*>(a.Qf) + ((size_t)h * a.M + m) * D + 4 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = to_f(q[i]);
    if (a.norm_qf) {
      float ss = qf[0] * qf[0] + qf[1] * qf[1] + qf[2] * qf[2] + qf[3] * qf[3];
      for (int o = 1; o < CPS; o <<= 1) ss += __shfl_xor(ss, o);
      const float r = norm_factor(ss, D, a.eps);
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] *= r;
    }
  }
  if (pg != 0) return;
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (st.A > -INFINITY) {
    z = st.num / st.den;
    lse = kLn2 * (st.A + __builtin_amdgcn_logf(st.den));
  }
  if (a.zmul) z = z * reinterpret_cast<const f32x4*>(a.zmul + (size_t)h * D)[c];
  const size_t o = ((size_t)bh * a.M + m) * D + 4 * c;
  if (a.Qout) {
    const float g = a.gate[h];
    *reinterpret_cast<f32x4*>(a.Qout + o) = f32x4{qf[0] + g * z[0], qf[1] + g * z[1], qf[2] + g * z[2], qf[3] + g * z[3]};
  } else {
    *reinterpret_cast<f32x4*>(a.Z + o) = z;
    if (a.L && c == 0) a.L[(size_t)bh * a.M + m] = lse;
  }
}

// ----------------------------------------------------------------------------
// Decode
// ----------------------------------------------------------------------------
struct DecArgs {
  const void* Q;   // [H,M,D] or [B,H,M,D], type QT
  const void* K;   // [B,H,N,D], type T
  const float* Z;  // [B,H,M,D]
  void* Y;         // [B,H,N,D], type T
  long long total; // nbh * N
  int q_batched, H, N, M, MB, nwg, bh0;
  float qscale;
  const float* qmul;  // [H, D] channel scale of the queries (the keys' N_a scale), or null
  float eps;          // key rows are N_0-normalised when the kernel's NK flag is set
  const float* kmax;  // [B H] largest squared key norm of each head (from its encode), or null
  // With the kernel's MRG flag, Z is not read: the staging merges the head's
  // split partials itself (the encode's plan: total etotal, enwg pieces, eWN
  // splits per piece, pmax slots per head), takes the head's key-norm maximum
  // from part_km (or null), and the workgroup holding the head's first token
  // writes Z and L to Zout and Lout (or null).
  const float* part_acc;  // [nbh][pmax][M][D]
  const float2* part_al;  // [nbh][pmax][M]
  const float* part_km;   // [nbh][pmax]
  float* Zout;            // [B,H,M,D]
  float* Lout;            // [B,H,M]
  long long etotal;
  int enwg, eWN, pmax;
  // statistics mode (the kernel's ST flag, bf16): instead of Y, per token
  // one record of 8 bf16 (see split3_record): the negated log2 of the
  // weight sum over the latents and the negated dY . Y, each as three parts
  const void* dY;     // [B,H,N,D], type T
  uint4* srec;        // [B,H,N]
};

// Z (features d0 .. d0 + 3 of latent m) and L of one head from its cnt
// split partials at slots pbase .. pbase + cnt - 1, folded in ascending order
// by the merge's rule; each batch of kMergeBatch splits is loaded before any
// of it is folded.
__device__ inline f32x4 merge_splits(const float* part_acc, const float2* part_al, size_t pbase, int cnt, int M, int D,
                                     int m, int d0, float& lse) {
  MergeState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int p0 = 0; p0 < cnt; p0 += kMergeBatch) {
    float2 v[kMergeBatch];
    f32x4 u[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int p = p0 + j;
      v[j] = make_float2(-INFINITY, 0.f);  // slots past cnt count as empty
      u[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p < cnt) {
        const size_t i = (pbase + p) * M + m;
        v[j] = part_al[i];
        u[j] = *reinterpret_cast<const f32x4*>(part_acc + i * D + d0);
      }
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) st = merge_fold(st, v[j].x, v[j].y, u[j]);
  }
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  lse = -INFINITY;
  if (st.A > -INFINITY) {
    z = st.num / st.den;
    lse = kLn2 * (st.A + __builtin_amdgcn_logf(st.den));
  }
  return z;
}

// Record of two float32 values x, y as 8 bf16: x = x0 + x1 + x2 and
// y = y0 + y1 + y2 (each part the bf16 rounding of what the previous parts
// leave, so the sum carries the float's full precision), as
// [x0, x1, x2, 0, y0, y1, y2, 0].  A matrix product whose other operand holds
// ones at those positions adds x or y to a result exactly.
__device__ inline uint4 split3_record(float x, float y) {
  bf16x8 r;
  float t = x;
#pragma unroll
  for (int i = 0; i < 3; ++i) { r[i] = (bf16)t; t -= (float)r[i]; }
  r[3] = (bf16)0.f;
  t = y;
#pragma unroll
  for (int i = 4; i < 7; ++i) { r[i] = (bf16)t; t -= (float)r[i]; }
  r[7] = (bf16)0.f;
  return *reinterpret_cast<uint4*>(&r);
}

template <typename T, int D> struct DecLds {
  static constexpr int E = 16 / sizeof(T);
  static constexpr int QST = D + E;
  // row stride of the transposed latents: 2 mod 4 dwords for bf16, so the 32
  // feature rows read by a wave's 8-byte PV operand loads hit distinct banks
  __host__ __device__ static size_t zst(int MB) { return (size_t)MB * 32 + 4; }
  static size_t bytes(int MB) { return ((size_t)MB * 32 * QST + (size_t)D * zst(MB)) * sizeof(T); }
};

// TAIL: M is not a multiple of 32, so the last latent block has rows past M
// that must not receive weight (compiled out for whole blocks).  NK: each
// token's key row is N_0-normalised in registers once per step (bf16).  ST:
// statistics mode for the backward (bf16): the log-normaliser of every
// token's softmax over the latents (log2 units, the queries' scaling) and
// the dot product of the token's output cotangent with its output.
// MBT > 0 fixes the number of latent blocks at compile time (a.MB == MBT), so
// the latent loop unrolls completely; 0 reads it from the arguments.  MRG:
// the staging merges the encode's split partials (see DecArgs).
//
// One workgroup of kDecWaves waves per compute unit (four per SIMD) shares a
// head's staged queries and latents.  Its waves take the piece's 32-token
// blocks from a counter in LDS as they finish the previous one, so all of them
// run to the end of the piece together: with several workgroups per compute
// unit the oldest ones are issued first, finish early and leave the last to
// run alone at one wave per SIMD.
// Piece `piece` of a.nwg (the workgroup's); smem: DecLds<T, D>::bytes(MB)
// of LDS, zred and qred: kDecWaves floats of LDS each, next_blk: one int of
// LDS (the next unclaimed 32-token block of the piece).
template <typename T, typename QT, int D, bool TAIL, bool NK, bool ST = false, int MBT = 0, bool MRG = false>
__device__ __attribute__((always_inline)) inline void decode_body(const DecArgs& a, int piece, unsigned char* smem,
                                                                  float* zred, float* qred, int& next_blk) {
  static_assert(!ST || sizeof(T) == 2, "statistics mode is bf16 only");
  // key rows N_0 on the fly: fp16 score operands (queries and keys; see
  // qk_mma_h), except in statistics mode, whose weights the backward forms
  // again from bf16 keys
  constexpr bool H = NK && !ST && sizeof(T) == 2;
  using L = DecLds<T, D>;
  const int MB = MBT > 0 ? MBT : a.MB, Mp = 32 * MB, M = a.M, N = a.N;
  T* qs = reinterpret_cast<T*>(smem);
  T* zt = qs + (size_t)Mp * L::QST;
  const int zst = (int)L::zst(MB);
  // the wave index is uniform: kept in a scalar register, block guards derived
  // from it become scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  constexpr bool mask_tail = TAIL;
  __builtin_assume(MB >= 1);

  long long x = piece_start(piece, a.total, a.nwg);
  const long long xe = piece_start(piece + 1, a.total, a.nwg);
  while (x < xe) {
    const int bhl = (int)(x / N);
    const long long hb = (long long)bhl * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int bh = a.bh0 + bhl;
    const int h = bh % a.H;

    // Stage this head's scaled queries (rows = latents) and transposed
    // latents.  Every 16-byte chunk of the head is loaded before the first
    // one is used, so staging costs one memory round trip rather than one per
    // element; rows M .. Mp-1 are zero.
    __syncthreads();
    const QT* Qh = reinterpret_cast<const QT*>(a.Q) + (size_t)(a.q_batched ? bh : h) * M * D;
    const float* Zh = a.Z + (size_t)bh * M * D;
    // MRG: the head's split slots, and whether this workgroup writes Z and L
    int cnt = 0;
    size_t pbase = 0;
    if constexpr (MRG) {
      cnt = (piece_of(hb + N - 1, a.etotal, a.enwg) - piece_of(hb, a.etotal, a.enwg) + 1) * a.eWN;
      pbase = (size_t)bhl * a.pmax;
    }
    const bool writer = MRG && n_lo == 0;
    float zmax = 0.f;
    float qerr2 = 0.f;  // largest squared rounding error of a staged query row
    {
      constexpr int QE = 16 / sizeof(QT);          // elements per 16-byte chunk
      constexpr int QJ = (256 * D / QE + kDecThreads - 1) / kDecThreads;  // chunks per thread at M = 256
      constexpr int ZJ = (256 * D / 4 + kDecThreads - 1) / kDecThreads;
      const int nq = M * D / QE, nz = M * D / 4;   // chunks of real rows
      const int pq = Mp * D / QE, pz = Mp * D / 4; // chunks including the zero rows
      // chunk offsets from an index opaque to the compiler, so they are
      // recomputed here rather than hoisted out of the head loop and spilled
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      uint4 qv[QJ], zv[ZJ];
#pragma unroll
      for (int j = 0; j < QJ; ++j) {
        const int c = tid + j * kDecThreads;
        qv[j] = reinterpret_cast<const uint4*>(Qh)[c < nq ? c : 0];
      }
      if constexpr (!MRG) {
#pragma unroll
        for (int j = 0; j < ZJ; ++j) {
          const int c = tid + j * kDecThreads;
          zv[j] = reinterpret_cast<const uint4*>(Zh)[c < nz ? c : 0];
        }
      }
#pragma unroll
      for (int j = 0; j < QJ; ++j) {
        const int c = tid + j * kDecThreads;
        float ce2 = 0.f;  // squared rounding error of these QE staged values
        if (c < pq) {
          const int m = c * QE / D, d0 = c * QE % D;
          const QT* src = reinterpret_cast<const QT*>(&qv[j]);
          float qm[QE];  // the channel scale of these QE features (16-byte aligned), or ones
          if (a.qmul) {
#pragma unroll
            for (int k = 0; k < QE / 4; ++k) {
              const f32x4 t = reinterpret_cast<const f32x4*>(a.qmul + (size_t)h * D + d0)[k];
#pragma unroll
              for (int i = 0; i < 4; ++i) qm[4 * k + i] = t[i];
            }
          } else {
#pragma unroll
            for (int i = 0; i < QE; ++i) qm[i] = 1.f;
          }
#pragma unroll
          for (int i = 0; i < QE; ++i) {
            const float q = (c < nq ? to_f(src[i]) * a.qscale : 0.f) * qm[i];
            T r;
            float rv;
            if constexpr (H) {
              r = h_bits(q);
              rv = h_val(r);
            } else {
              r = from_f<T>(q);
              rv = to_f(r);
            }
            qs[m * L::QST + d0 + i] = r;
            ce2 += (q - rv) * (q - rv);
          }
        }
        // the D / QE chunks of a row sit in consecutive, aligned lanes
#pragma unroll
        for (int o = 1; o < D / QE; o <<= 1) ce2 += __shfl_xor(ce2, o);
        qerr2 = fmaxf(qerr2, ce2);
      }
#pragma unroll
      for (int j = 0; j < ZJ; ++j) {
        const int c = tid + j * kDecThreads;
        if (c < pz) {
          const int m = c * 4 / D, d0 = c * 4 % D;
          f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
          if (c < nz) {
            if constexpr (MRG) {
              float lse;
              z4 = merge_splits(a.part_acc, a.part_al, pbase, cnt, M, D, m, d0, lse);
              if (writer) {
                *reinterpret_cast<f32x4*>(a.Zout + ((size_t)bh * M + m) * D + d0) = z4;
                if (a.Lout && d0 == 0) a.Lout[(size_t)bh * M + m] = lse;
              }
            } else {
              z4 = *reinterpret_cast<const f32x4*>(&zv[j]);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            zt[(d0 + i) * zst + m] = from_f<T>(z4[i]);
            zmax = fmaxf(zmax, fabsf(z4[i]));
          }
        }
      }
    }
    // |Y accumulator| <= (sum of weights) * max |z|: a token block whose
    // weight sum stays below zlim cannot have overflowed (see fast_failed)
    zmax = wave_max(zmax);
    qerr2 = wave_max(qerr2);
    if (lane == 0) { zred[wave] = zmax; qred[wave] = qerr2; }
    // wave w starts with block w; the counter hands out the rest
    if (threadIdx.x == 0) next_blk = kDecWaves;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) { zmax = fmaxf(zmax, zred[w]); qerr2 = fmaxf(qerr2, qred[w]); }
    const float zlim = 1.329228e36f / fmaxf(zmax * 1.01f, 1.f);  // 2^120 / max|z|
    // a token block keeps the fast loop's result only if every score it
    // forms is within kScoreErr of the exact one: |k_n|^2 <= klim2.  When the
    // head's encode found no key beyond that (with 1% for the rounding of
    // keys normalised there and here), no block needs the check.
    const float klim2 = qerr2 > 0.f ? kScoreErr2 / qerr2 : INFINITY;
    float khead = INFINITY;  // the head's largest squared key norm, if known
    if constexpr (MRG) {
      if (a.part_km) {
        khead = 0.f;
        for (int p = lane; p < cnt; p += 64) khead = fmaxf(khead, a.part_km[pbase + p]);
        khead = wave_max(khead);
      }
    } else {
      if (a.kmax) khead = a.kmax[bh];
    }
    const bool kcheck = !(khead * 1.01f <= klim2);

    const T* Kh = reinterpret_cast<const T*>(a.K) + (size_t)bh * N * D;
    T* Yh = reinterpret_cast<T*>(a.Y) + (size_t)bh * N * D;
    // Block b holds tokens n_lo + 32 b + [0, 32); the wave claims its next
    // block when it starts one and fetches that block's key rows while the
    // current one is decoded.  Lanes past the piece read its last row instead:
    // their outputs are not stored and their scores only reach their own
    // column.
    const int nblk = (n_hi - n_lo + 31) / 32;
    int b = wave;
    int t0 = n_lo + 32 * b;
    QKOp<T, D> kop;
    load_op<D>(kop, Kh + (size_t)(t0 + li < n_hi ? t0 + li : n_hi - 1) * D, g);
    // Settle these keys before the loop: inside it the compiler would place
    // the wait for them after the prefetch and so also wait for the prefetch.
#pragma unroll
    for (int st = 0; st < (int)(sizeof(kop.v) / sizeof(kop.v[0])); ++st) asm volatile("" : "+v"(kop.v[st]));
    const f32x16 zero16 = {};
    while (b < nblk) {
      if constexpr (NK) norm_op<D, H>(kop, a.eps);
      int bn = 0;
      if (lane == 0) bn = atomicAdd(&next_blk, 1);
      bn = __builtin_amdgcn_readfirstlane(bn);
      QKOp<T, D> knext;
      {
        const int tn = n_lo + 32 * bn + li;
        load_op<D>(knext, Kh + (size_t)(tn < n_hi ? tn : n_hi - 1) * D, g);
      }
      f32x16 acc;
      float lsum = 0.f, den, shift = 0.f;
      if constexpr (sizeof(T) == 2) {
        // Fast path: unshifted weights exp2(score) (see fast_ok).  The
        // scores of latent block mb + 1 go to the MFMA unit before the
        // weights of block mb are exponentiated, so within the wave the
        // matrix products run under the exponentials.
        RowSum<D> wsum(lane);
        // This lane's LDS rows, recomputed for every token block from an
        // index opaque to the compiler: held across the block loop they are
        // spilled, and the reload's wait would also wait for the key prefetch.
        int lid = threadIdx.x;
        asm volatile("" : "+v"(lid));
        const T* qrow = qs + (lid & 31) * L::QST;
        const T* zrow = zt + (lid & 31) * zst;
        auto scores = [&](int mb) {
          QKOp<T, D> qop;
          load_op<D>(qop, qrow + mb * 32 * L::QST, g);
          return qk_mma_sel<H, D>(qop, kop, zero16);
        };
        auto consume = [&](f32x16 sc, int mb, const f32x16& from) {
          PVOp<T> zop;
          if (li < D) load_pv(zop, zrow + mb * 32, g);
          else pad_pv(zop, li, D);
          if (mask_tail && mb == MB - 1) mask_rows(sc, M - mb * 32, g);
          bf16x8 b0, b1;
          wsum.add(sc, b0, b1);
          acc = pv_mma(zop, b0, b1, from);
        };
        f32x16 sa = scores(0), sb;
        if (MB > 1) sb = scores(1);
        consume(sa, 0, zero16);
        int mb = 1;
        constexpr int kUnroll = MBT > 0 ? MBT : 1;
#pragma unroll kUnroll
        for (; mb + 2 < MB; mb += 2) {  // block mb is in sb
          sa = scores(mb + 1);
          consume(sb, mb, acc);
          sb = scores(mb + 2);
          consume(sa, mb + 1, acc);
        }
        if (mb + 1 < MB) {
          sa = scores(mb + 1);
          consume(sb, mb, acc);
          consume(sa, mb + 1, acc);
        } else if (mb < MB) {
          consume(sb, mb, acc);
        }
        den = wsum.total(li, acc);
        // |Y accumulator| <= den * max |z| stays below 2^120 when den <= zlim;
        // the staged queries' rounding moves no score of a key with
        // |k|^2 <= klim2 by more than kScoreErr
        const bool redo = !fast_ok(den) || den > zlim || (kcheck && row_norm2<D, H>(kop) > klim2);
        if (__builtin_amdgcn_ballot_w64(redo) != 0) {
          // careful redo of this token block: exact scores (the queries read
          // again and split into bf16 hi + lo) and the exact maximum of
          // every latent block
          f32x16 negs = zero16;
          bool started = false;
          acc = zero16;
          lsum = 0.f;
          const float* qm = a.qmul ? a.qmul + (size_t)h * D : nullptr;
          QKOp<T, D> kx = kop;  // bf16 keys
          if constexpr (H) {  // this lane's key row again, N_0 in bf16
            load_op<D>(kx, Kh + (size_t)(t0 + li < n_hi ? t0 + li : n_hi - 1) * D, g);
            norm_op<D>(kx, a.eps);
          }
          int mc = 0;
          do {
            const int m = mc * 32 + li;
            QKOp<T, D> qhi, qlo;
            load_q_row<D>(qhi, &qlo, Qh + (size_t)(m < M ? m : M - 1) * D, g, a.qscale, false, 0.f, qm, nullptr);
            if (m >= M) { zero_op<D>(qhi); zero_op<D>(qlo); }
            PVOp<T> zop;
            if (li < D) load_pv(zop, zt + li * zst + mc * 32, g);
            else ones_pv(zop, li, D);
            f32x16 sc = qk_mma<D>(qlo, kx, qk_mma<D>(qhi, kx, negs));
            if (mask_tail && mc == MB - 1) mask_rows(sc, M - mc * 32, g);
            online_step(sc, negs, started, lsum, acc);
            bf16x8 b0, b1;
            lsum += pack_exps(sc, b0, b1);
            acc = pv_mma(zop, b0, b1, acc);
          } while (++mc < MB);
          den = pair_sum(lsum);
          shift = -negs[0];
        }
      } else {
        f32x16 negs = zero16;
        bool started = false;
        acc = zero16;
        for (int mb = 0; mb < MB; ++mb) {
          QKOp<T, D> qop;
          load_op<D>(qop, qs + (mb * 32 + li) * L::QST, g);
          PVOp<T> zop;
          if (li < D) load_pv(zop, zt + li * zst + mb * 32, g);
          else ones_pv(zop, li, D);
          f32x16 sc = qk_mma<D>(qop, kop, negs);
          if (mask_tail && mb == MB - 1) mask_rows(sc, M - mb * 32, g);
          online_step(sc, negs, started, lsum, acc);
          acc = pv_accum<D>(zop, sc, acc, lsum);
        }
        den = col_sum<T, D>(lsum, acc);
      }
      // Lanes past the piece decoded the piece's last key row, so their
      // output is bitwise that of token n_hi - 1: they store it there too.
      // The stores are unconditional on purpose: inside a divergent branch
      // the compiler's wait for the prefetched keys below would also wait
      // for them to reach memory.
      const int n = t0 + li < n_hi ? t0 + li : n_hi - 1;
      const float inv = __builtin_amdgcn_rcpf(den);
      if constexpr (ST) {
        const T* dy = reinterpret_cast<const T*>(a.dY) + ((size_t)bh * N + n) * D;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (8 * c + 4 * g < D) {
            const bf16x4 v = *reinterpret_cast<const bf16x4*>(dy + 8 * c + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) part += acc[4 * c + i] * (float)v[i];
          }
        }
        const float dot = pair_sum(part) * inv;
        // both lanes of the pair store the same record: a store in a divergent
        // branch would make the wait for the prefetched keys cover it
        a.srec[(size_t)bh * N + n] = split3_record(-(shift + __builtin_amdgcn_logf(den)), -dot);
      } else {
        T* dst = Yh + (size_t)n * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (8 * c + 4 * g < D) {
            if constexpr (sizeof(T) == 2) {
              bf16x4 v;
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[4 * c + i] * inv);
              *reinterpret_cast<bf16x4*>(dst + 8 * c + 4 * g) = v;
            } else {
              f32x4 v;
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = acc[4 * c + i] * inv;
              *reinterpret_cast<f32x4*>(dst + 8 * c + 4 * g) = v;
            }
          }
        }
      }
      kop = knext;
      b = bn;
      t0 = n_lo + 32 * b;
    }
    x = hb + n_hi;
  }
}

template <typename T, typename QT, int D, bool TAIL, bool NK, bool ST = false, int MBT = 0, bool MRG = false>
__global__ void __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) decode_kernel(DecArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float zred[kDecWaves], qred[kDecWaves];
  __shared__ int next_blk;
  decode_body<T, QT, D, TAIL, NK, ST, MBT, MRG>(a, blockIdx.x, smem, zred, qred, next_blk);
}

// ----------------------------------------------------------------------------
// FLARE and FLARE++ forward with one workgroup per head
// ----------------------------------------------------------------------------
// With many heads of a few thousand tokens, the launches of the forward
// (FLARE++: synthesis encode, blended merge, routing encode, merge, decode;
// FLARE: the last three) spend much of their time filling and draining the
// chip between steps.  Here one workgroup of kHeadWaves waves takes a whole
// head through the steps, with workgroup barriers in place of the kernel
// boundaries: the head is one piece of WN splits (one per token lane of
// waves), whose partials stay in LDS and are merged there by the whole
// workgroup; the blended queries and the latents pass through their buffers
// to the next step.  The encodes and the decode run the device code of their
// own kernels.
constexpr int kHeadWaves = 16;
static_assert(kHeadWaves == kDecWaves, "the decode step runs with the decode's wave count");

struct HeadArgs {
  EncArgs se, re;      // synthesis encode (bf16 seeds, FLARE++), routing encode
  DecArgs d;           // decode
  const bf16* Qf;      // [H,M,D] fixed queries of the blend (FLARE++)
  const float* gate;   // [H]
  float* Qout;         // [B,H,M,D] blended queries (the routing queries)
  float* Z;            // [B,H,M,D]
  float* L;            // [B,H,M]
  int H, nbh;          // heads per batch entry, B H
};

// Token lanes (splits) of the encode steps for MB latent blocks, the tile rows
// that give each of them two 32-token blocks per tile (the scores of the
// second go to the matrix core before the first one's weights are formed),
// and the dynamic LDS: the encode's tiles; once an encode has consumed them,
// its split partials [WN][M][D] and their (shift, sum) [WN][M]; in the decode
// its staged queries and latents.
template <int MB> constexpr int head_wn() { return kHeadWaves / MB; }
template <int MB> constexpr int head_rows() { return 64 * head_wn<MB>(); }
template <int MB> constexpr size_t head_tile_bytes() { return (size_t)4 * head_rows<MB>() * 32 * sizeof(bf16); }
template <int MB> constexpr size_t head_part_bytes() {
  return (size_t)head_wn<MB>() * 32 * MB * (32 * sizeof(float) + sizeof(float2));
}
template <int MB> constexpr size_t head_lds() {
  return head_tile_bytes<MB>() > head_part_bytes<MB>() ? head_tile_bytes<MB>() : head_part_bytes<MB>();
}

// The merge of one head's split partials from LDS (lacc [WN][M][D], lal
// [WN][M]) for latent m, features 4 c .. 4 c + 3: the splits are folded in
// ascending order as in merge_kernel.  Returns Z's four features and sets L.
template <int WN, int D>
__device__ inline f32x4 merge_lds(const float* lacc, const float2* lal, int M, int m, int c, float& lse) {
  MergeState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int p = 0; p < WN; ++p) {
    const float2 al = lal[p * M + m];
    st = merge_fold(st, al.x, al.y, reinterpret_cast<const f32x4*>(lacc + ((size_t)p * M + m) * D)[c]);
  }
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  lse = -INFINITY;
  if (st.A > -INFINITY) {
    z = st.num / st.den;
    lse = kLn2 * (st.A + __builtin_amdgcn_logf(st.den));
  }
  return z;
}

// D = 32, MB latent blocks (M = 32 MB), bf16 keys and values; one head per
// workgroup (blockIdx.x = head); dynamic LDS of head_lds<MB>() bytes.  Thread
// t merges latent t / 8, features 4 (t % 8) .. + 3.  PP: the FLARE++ forward,
// whose routing queries are the float32 blended ones it writes to a.Qout;
// else the FLARE forward with the bf16 queries of a.re.
template <int MB, bool PP>
__global__ void __launch_bounds__(kHeadWaves * 64) head_kernel(HeadArgs a) {
  using RQ = typename std::conditional<PP, float, bf16>::type;  // routing query element type
  constexpr int D = 32, M = 32 * MB, WN = head_wn<MB>(), ROWS = head_rows<MB>();
  static_assert(M * D / 4 <= kHeadWaves * 64, "one latent chunk per thread");
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[2 * kHeadWaves];
  __shared__ int next_blk;
  bf16* const tiles = reinterpret_cast<bf16*>(smem);
  float* const lacc = reinterpret_cast<float*>(smem);  // the tiles' space: written once the tiles are consumed
  float2* const lal = reinterpret_cast<float2*>(lacc + WN * M * D);
  const int bh = blockIdx.x, h = bh % a.H;
  const int m = threadIdx.x / (D / 4), c = threadIdx.x % (D / 4);
  const bool mine = m < M;
  const size_t o = ((size_t)bh * M + m) * D + 4 * c;

  if constexpr (PP) {
    encode_dma_body<bf16, D, kHeadWaves, WN, false, ROWS, true>(a.se, bh, tiles, red, lacc, lal);
    float qf[4] = {0.f, 0.f, 0.f, 0.f};
    if (mine) {
      const bf16* q = a.Qf + ((size_t)h * M + m) * D + 4 * c;
#pragma unroll
      for (int i = 0; i < 4; ++i) qf[i] = (float)q[i];
    }
    const float g = a.gate[h];
    __syncthreads();  // the synthesis partials are in LDS
    if (mine) {
      float lse;
      const f32x4 z = merge_lds<WN, D>(lacc, lal, M, m, c, lse);
      *reinterpret_cast<f32x4*>(a.Qout + o) =
          f32x4{qf[0] + g * z[0], qf[1] + g * z[1], qf[2] + g * z[2], qf[3] + g * z[3]};
    }
    __syncthreads();  // the blended queries are written, the partials read
  }
  encode_dma_body<RQ, D, kHeadWaves, WN, false, ROWS, true>(a.re, bh, tiles, red, lacc, lal);
  __syncthreads();
  if (mine) {
    float lse;
    const f32x4 z = merge_lds<WN, D>(lacc, lal, M, m, c, lse);
    *reinterpret_cast<f32x4*>(a.Z + o) = z;
    if (c == 0) a.L[(size_t)bh * M + m] = lse;
  }
  __syncthreads();  // Z is written
  decode_body<bf16, RQ, D, false, false, false, MB>(a.d, bh, smem, red, red + kHeadWaves, next_blk);
}

// ----------------------------------------------------------------------------
// FLARE++ encodes with one workgroup per (head, latent block)
// ----------------------------------------------------------------------------
// The encode of a latent needs only that latent's query, so a head's latent
// blocks can be encoded apart, each over all of the head's tokens: then no
// split partials leave the workgroup and no merge launch follows, and a head
// of M = 32 MB latents spreads over MB compute units.  One workgroup runs the
// synthesis encode, the blend and the routing encode of one latent block
// (the routing encode of a latent needs only its own blended query); the
// decode, which needs all of a head's latents, follows as its own launch.  A
// workgroup of kHeadWaves waves takes the block's 32 latents with all waves
// as token lanes.
constexpr int kLatRows = 32 * kHeadWaves;  // tokens per tile: one 32-token block per wave
constexpr size_t kLatTileBytes = (size_t)4 * kLatRows * 32 * sizeof(bf16);
constexpr size_t kLatPartBytes = (size_t)kHeadWaves * 32 * (32 * sizeof(float) + sizeof(float2));
constexpr size_t kLatLds = kLatTileBytes > kLatPartBytes ? kLatTileBytes : kLatPartBytes;

// D = 32, bf16 keys and values; workgroup w takes head w % nbh and latent
// block w / nbh (latents 32 (w / nbh) .. + 31), so the workgroups of a head
// are nbh apart; dynamic LDS of kLatLds bytes.  Thread t < 256 merges latent
// t / 8 of the block, features 4 (t % 8) .. + 3.  Writes the blended queries
// a.Qout, Z and L of its latents, and the head's largest squared routing-key
// norm to the routing encode's part_km (block 0).
__global__ void __launch_bounds__(kHeadWaves * 64) latent_kernel(HeadArgs a) {
  constexpr int D = 32, WN = kHeadWaves, NC = 32 * D / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[kHeadWaves];
  bf16* const tiles = reinterpret_cast<bf16*>(smem);
  float* const lacc = reinterpret_cast<float*>(smem);  // the tiles' space: written once the tiles are consumed
  float2* const lal = reinterpret_cast<float2*>(lacc + WN * 32 * D);
  const int mb = (int)blockIdx.x / a.nbh, bh = (int)blockIdx.x - mb * a.nbh, h = bh % a.H, M = a.re.M;
  const int ml = threadIdx.x / (D / 4), c = threadIdx.x % (D / 4), m = 32 * mb + ml;
  const bool mine = threadIdx.x < NC && m < M;
  const size_t o = ((size_t)bh * M + m) * D + 4 * c;

  EncArgs se = a.se;
  se.m0 = 32 * mb;
  encode_dma_body<bf16, D, kHeadWaves, WN, false, kLatRows, true>(se, bh, tiles, red, lacc, lal);
  float qf[4] = {0.f, 0.f, 0.f, 0.f};
  if (mine) {
    const bf16* q = a.Qf + ((size_t)h * M + m) * D + 4 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) qf[i] = (float)q[i];
  }
  const float g = a.gate[h];
  __syncthreads();  // the synthesis partials are in LDS
  if (mine) {
    float lse;
    const f32x4 z = merge_lds<WN, D>(lacc, lal, 32, ml, c, lse);
    *reinterpret_cast<f32x4*>(a.Qout + o) = f32x4{qf[0] + g * z[0], qf[1] + g * z[1], qf[2] + g * z[2], qf[3] + g * z[3]};
  }
  __syncthreads();  // the block's blended queries are written, the partials read
  EncArgs re = a.re;
  re.m0 = 32 * mb;
  if (mb != 0) re.part_km = nullptr;  // the head's key-norm maximum: written once
  encode_dma_body<float, D, kHeadWaves, WN, false, kLatRows, true>(re, bh, tiles, red, lacc, lal);
  __syncthreads();
  if (mine) {
    float lse;
    const f32x4 z = merge_lds<WN, D>(lacc, lal, 32, ml, c, lse);
    *reinterpret_cast<f32x4*>(a.Z + o) = z;
    if (c == 0) a.L[(size_t)bh * M + m] = lse;
  }
}

// ----------------------------------------------------------------------------
// Host side: planning, validation, launches
// ----------------------------------------------------------------------------
struct Dev {
  int cus = 0;
  size_t lds_max = 0;
};

int query_dev(Dev& d) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLARE_ERR_HIP;
  int cus = 0, lds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FLARE_ERR_HIP;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return FLARE_ERR_HIP;
  d.cus = cus > 0 ? cus : 1;
  d.lds_max = (size_t)lds;
  return FLARE_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// Launch a kernel and return that launch's own status.  (hipGetLastError
// after a launch would also return, and clear, an error left pending by an
// earlier, unrelated call on this thread.)
template <typename... P, typename... A, size_t... I>
int launch_impl(void (*fn)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, std::index_sequence<I...>,
                A&&... args) {
  std::tuple<P...> vals(std::forward<A>(args)...);
  void* argv[] = {(void*)&std::get<I>(vals)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, argv, lds, st) == hipSuccess ? FLARE_OK
                                                                                                      : FLARE_ERR_HIP;
}
template <typename... P, typename... A>
int launch(void (*fn)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A&&... args) {
  return launch_impl(fn, grid, block, lds, st, std::index_sequence_for<P...>{}, std::forward<A>(args)...);
}

// Latent blocks of 32: padded to 1, 2, 4 or 8 so that waves split them evenly.
inline int latent_blocks(int M) {
  int mb = (int)cdiv(M, 32);
  int p = 1;
  while (p < mb) p *= 2;
  return p;
}

struct EncPlan {
  int G, MBW, WN, NW, nwg, pmax;
  long long total;
};

// Resident waves per compute unit the encode grid is sized for: 16, or 8 when
// there are at most kEncSmallTokensPerCu tokens per compute unit (there the
// longer pieces and the fewer splits to merge measured 4-6% faster at the
// PDE-mesh and point-cloud workloads, and 16 waves 2-4% faster at the
// million-token one).  The decode's workgroups per compute unit.
constexpr int kEncWavesPerCu = 16, kEncWavesPerCuSmall = 8;
constexpr long long kEncSmallTokensPerCu = 8192;
constexpr int kDecWgPerCu = 1;

// bf16: one 32-latent block per wave, max(4, blocks) waves per workgroup.
// f32: up to two latent blocks per wave, 4 waves per workgroup.
EncPlan plan_encode(const Dev& dev, int nbh, int N, int M, int dtype) {
  EncPlan p{};
  const int mbp = latent_blocks(M);
  if (dtype == FLARE_BF16) {
    p.MBW = 1;
    p.G = mbp;
    p.NW = mbp > 4 ? mbp : 4;
  } else {
    p.MBW = mbp >= 2 ? 2 : 1;
    p.G = mbp / p.MBW;
    p.NW = 4;
  }
  p.WN = p.NW / p.G;
  p.total = (long long)nbh * N;
  const int wpc = p.total <= (long long)dev.cus * kEncSmallTokensPerCu ? kEncWavesPerCuSmall : kEncWavesPerCu;
  long long want = (long long)dev.cus * wpc / p.NW;
  long long maxw = cdiv(p.total, kTile);
  p.nwg = (int)(want < maxw ? want : maxw);
  if (p.nwg < 1) p.nwg = 1;
  int pm = 1;
  for (int bhl = 0; bhl < nbh && N > 0; ++bhl) {
    const long long hb = (long long)bhl * N;
    const int c = piece_of(hb + N - 1, p.total, p.nwg) - piece_of(hb, p.total, p.nwg) + 1;
    if (c > pm) pm = c;
  }
  p.pmax = pm * p.WN;
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int check_common(int B, int H, int N, int M, int D, int dtype, int q_batched) {
  if (B < 1 || H < 1 || N < 0 || M < 1) return FLARE_ERR_INVALID_ARG;
  if (q_batched != 0 && q_batched != 1) return FLARE_ERR_INVALID_ARG;
  if (dtype != FLARE_F32 && dtype != FLARE_BF16) return FLARE_ERR_UNSUPPORTED;
  if (D != 16 && D != 32) return FLARE_ERR_UNSUPPORTED;
  if (M > 256) return FLARE_ERR_UNSUPPORTED;
  if ((long long)B * H * (long long)(N > 0 ? N : 1) >= (1LL << 31)) return FLARE_ERR_UNSUPPORTED;
  if ((long long)B * H * M * D >= (1LL << 31)) return FLARE_ERR_UNSUPPORTED;
  return FLARE_OK;
}

template <typename QT, int D, int NW, int WN, bool NK, bool H>
int launch_encode_dma(const EncArgs& a, hipStream_t st) {
  return launch(encode_dma_kernel<QT, D, NW, WN, NK, H>, dim3(a.nwg), dim3(NW * 64), 0, st, a);
}

template <typename QT, int D, bool NK, bool H = false>
int launch_encode_bf16_dk(const EncArgs& a, int NW, int WN, hipStream_t st) {
  if (NW == 8 && WN == 1) return launch_encode_dma<QT, D, 8, 1, NK, H>(a, st);
  if (NW != 4) return FLARE_ERR_UNSUPPORTED;  // no kernel for this split plan
  if (WN == 4) return launch_encode_dma<QT, D, 4, 4, NK, H>(a, st);
  if (WN == 2) return launch_encode_dma<QT, D, 4, 2, NK, H>(a, st);
  return launch_encode_dma<QT, D, 4, 1, NK, H>(a, st);
}

// With key rows N_0 and separate values the scores take fp16 operands (the
// normalised keys and the queries; see qk_mma_h).  Values that alias the keys
// are normalised in the same tile and stay bf16 for the value products.
template <typename QT>
int launch_encode_bf16(const EncArgs& a, int D, int NW, int WN, bool nk, hipStream_t st) {
  if (nk && !a.v_alias)
    return D == 16 ? launch_encode_bf16_dk<QT, 16, true, true>(a, NW, WN, st)
                   : launch_encode_bf16_dk<QT, 32, true, true>(a, NW, WN, st);
  if (nk)
    return D == 16 ? launch_encode_bf16_dk<QT, 16, true>(a, NW, WN, st)
                   : launch_encode_bf16_dk<QT, 32, true>(a, NW, WN, st);
  return D == 16 ? launch_encode_bf16_dk<QT, 16, false>(a, NW, WN, st)
                 : launch_encode_bf16_dk<QT, 32, false>(a, NW, WN, st);
}

// Input normalisations of one launch sequence (FLARE++ paper, Table 2):
// query rows N_0 (norm_q) and channel scales qmul0, qmul1 ([H, D] or null),
// key rows N_0 (norm_k), epsilon.  Supported with bf16 keys and values.
struct Norms {
  int norm_q = 0;
  const float* qmul0 = nullptr;
  const float* qmul1 = nullptr;
  bool norm_k = false;
  float eps = 0.f;
};

template <int D, int MBW>
int launch_encode_f32(const EncArgs& a, hipStream_t st) {
  const size_t lds = EncLds<float, D>::bytes;
  return launch(encode_kernel<float, float, D, MBW>, dim3(a.nwg), dim3(kThreads), lds, st, a);
}

EncArgs encode_args(const void* Q, int q_batched, const void* K, const void* V, int bh0, int H, int N, int M,
                    float qscale, float* part_acc, float2* part_al, const EncPlan& p, const Norms& nm,
                    float* part_km) {
  EncArgs a;
  a.Q = Q; a.K = K; a.V = V;
  a.part_acc = part_acc; a.part_al = part_al; a.part_km = part_km;
  a.total = p.total;
  a.q_batched = q_batched; a.v_alias = (K == V); a.H = H; a.N = N; a.M = M;
  a.G = p.G; a.nwg = p.nwg; a.pmax = p.pmax; a.bh0 = bh0;
  a.qscale = qscale;
  a.norm_q = nm.norm_q; a.qmul0 = nm.qmul0; a.qmul1 = nm.qmul1; a.eps = nm.eps;
  return a;
}

// qtype: element type of Q (FLARE_F32 or FLARE_BF16); dtype: of K and V.
int launch_encode(const void* Q, int qtype, int q_batched, const void* K, const void* V, int bh0, int H, int N,
                  int M, int D, int dtype, float qscale, float* part_acc, float2* part_al, const EncPlan& p,
                  const Norms& nm, hipStream_t st, float* part_km = nullptr) {
  const EncArgs a = encode_args(Q, q_batched, K, V, bh0, H, N, M, qscale, part_acc, part_al, p, nm, part_km);
  if (dtype == FLARE_BF16) {
    if (qtype == FLARE_BF16) return launch_encode_bf16<bf16>(a, D, p.NW, p.WN, nm.norm_k, st);
    return launch_encode_bf16<float>(a, D, p.NW, p.WN, nm.norm_k, st);
  }
  if (nm.norm_q || nm.qmul0 || nm.qmul1 || nm.norm_k) return FLARE_ERR_UNSUPPORTED;
  if (qtype != FLARE_F32) return FLARE_ERR_UNSUPPORTED;
  if (D == 16) return p.MBW == 2 ? launch_encode_f32<16, 2>(a, st) : launch_encode_f32<16, 1>(a, st);
  return p.MBW == 2 ? launch_encode_f32<32, 2>(a, st) : launch_encode_f32<32, 1>(a, st);
}

MergeArgs merge_args(const EncPlan& p, const float* part_acc, const float2* part_al, int bh0, int nbh, int H,
                     int N, int M, int D, float* Z, float* L, const void* Qf, const float* gate, float* Qout,
                     int norm_qf, const float* zmul, float eps, const float* part_km, float* kmax) {
  MergeArgs a;
  a.part_acc = part_acc; a.part_al = part_al;
  a.part_km = part_km; a.kmax = part_km ? kmax : nullptr;
  a.Z = Z; a.L = L; a.Qf = Qf; a.gate = gate; a.Qout = Qout;
  a.norm_qf = norm_qf; a.zmul = zmul; a.eps = eps;
  a.total = p.total;
  a.N = N; a.M = M; a.D = D; a.H = H; a.WN = p.WN; a.nwg = p.nwg; a.pmax = p.pmax; a.bh0 = bh0; a.nbh = nbh;
  return a;
}

int launch_merge(const EncPlan& p, const float* part_acc, const float2* part_al, int bh0, int nbh, int H, int N,
                 int M, int D, float* Z, float* L, const void* Qf, int qftype, const float* gate, float* Qout,
                 int norm_qf, const float* zmul, float eps, hipStream_t st, const float* part_km = nullptr,
                 float* kmax = nullptr) {
  const MergeArgs a = merge_args(p, part_acc, part_al, bh0, nbh, H, N, M, D, Z, L, Qf, gate, Qout, norm_qf, zmul,
                                 eps, part_km, kmax);
  const dim3 grid((unsigned)cdiv((long long)nbh * M, kThreads / 64));
  if (qftype == FLARE_BF16) return launch(merge_kernel<bf16>, grid, dim3(kThreads), 0, st, a);
  return launch(merge_kernel<float>, grid, dim3(kThreads), 0, st, a);
}

template <typename T, typename QT, int D, bool TAIL, bool NK, bool ST = false, int MBT = 0, bool MRG = false>
int launch_decode_k(const DecArgs& a, size_t lds, hipStream_t st) {
  const void* fn = (const void*)decode_kernel<T, QT, D, TAIL, NK, ST, MBT, MRG>;
  if (lds > 65536) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return FLARE_ERR_HIP;
  }
  return launch(decode_kernel<T, QT, D, TAIL, NK, ST, MBT, MRG>, dim3(a.nwg), dim3(kDecThreads), lds, st, a);
}

// bf16 decode without a latent tail: 2, 4 or 8 latent blocks (M = 64, 128,
// 256) get a fully unrolled latent loop.
template <typename T, typename QT, int D, bool NK, bool ST = false>
int launch_decode_mb(const DecArgs& a, size_t lds, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    switch (a.MB) {
      case 2: return launch_decode_k<T, QT, D, false, NK, ST, 2>(a, lds, st);
      case 4: return launch_decode_k<T, QT, D, false, NK, ST, 4>(a, lds, st);
      case 8: return launch_decode_k<T, QT, D, false, NK, ST, 8>(a, lds, st);
      default: break;
    }
  }
  return launch_decode_k<T, QT, D, false, NK, ST>(a, lds, st);
}

template <typename T, typename QT, int D>
int launch_decode_t(const DecArgs& a, size_t lds, bool nk, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (nk)
      return (a.M & 31) ? launch_decode_k<T, QT, D, true, true>(a, lds, st)
                        : launch_decode_mb<T, QT, D, true>(a, lds, st);
  } else {
    if (nk) return FLARE_ERR_UNSUPPORTED;
  }
  return (a.M & 31) ? launch_decode_k<T, QT, D, true, false>(a, lds, st)
                    : launch_decode_mb<T, QT, D, false>(a, lds, st);
}

size_t decode_lds(int dtype, int D, int M) {
  const int MB = (int)cdiv(M, 32);
  if (dtype == FLARE_BF16) return D == 16 ? DecLds<bf16, 16>::bytes(MB) : DecLds<bf16, 32>::bytes(MB);
  return D == 16 ? DecLds<float, 16>::bytes(MB) : DecLds<float, 32>::bytes(MB);
}

// The encode's split partials for a decode that merges them in its staging
// (the kernel's MRG flag), with Z and L written by the first workgroup of
// each head.
struct DecMerge {
  const EncPlan* p = nullptr;
  const float* part_acc = nullptr;
  const float2* part_al = nullptr;
  const float* part_km = nullptr;
  float* Z = nullptr;
  float* L = nullptr;
};

// Whether the decode merges the splits itself: bf16 at M = 256 without key
// norms, with at least 16384 (head, latent) pairs and at most 16 splits per
// head.  The merge kernel takes one wave per pair, so its time grows with
// the pairs; the decode's staging instead folds a head's splits in about two
// memory round trips per workgroup.  (With few pairs or many splits the
// separate merge was measured faster: at the PDE-mesh and M = 64 point-cloud
// workloads, and at the million-token one.)
bool decode_merges(const EncPlan& p, int BH, int N, int M, int dtype, const Norms& nm) {
  return dtype == FLARE_BF16 && M == 256 && !nm.norm_k && N > 0 && (long long)BH * M >= 16384 && p.pmax <= 16;
}

// nm.norm_k: N_0 of the key rows; nm.qmul1: channel scale of the queries.
int launch_decode(const Dev& dev, const void* Q, int qtype, int q_batched, const void* K, const float* Z, void* Y,
                  int bh0, int nbh, int H, int N, int M, int D, int dtype, float qscale, const Norms& nm,
                  hipStream_t st, const float* kmax = nullptr, const DecMerge* mg = nullptr) {
  if (N == 0) return FLARE_OK;
  DecArgs a{};
  a.kmax = kmax;
  a.Q = Q; a.K = K; a.Z = Z; a.Y = Y;
  a.total = (long long)nbh * N;
  a.q_batched = q_batched; a.H = H; a.N = N; a.M = M; a.MB = (int)cdiv(M, 32); a.bh0 = bh0;
  a.qscale = qscale;
  a.qmul = nm.qmul1; a.eps = nm.eps;
  const bool nk = nm.norm_k;
  long long want = (long long)dev.cus * kDecWgPerCu;
  long long maxw = cdiv(a.total, 32);
  a.nwg = (int)(want < maxw ? want : maxw);
  const size_t lds = decode_lds(dtype, D, M);
  if (lds > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  if (mg) {  // decode_merges holds: bf16, M = 256 (8 whole latent blocks), no key norms
    a.part_acc = mg->part_acc; a.part_al = mg->part_al; a.part_km = mg->part_km;
    a.Zout = mg->Z; a.Lout = mg->L;
    a.etotal = mg->p->total; a.enwg = mg->p->nwg; a.eWN = mg->p->WN; a.pmax = mg->p->pmax;
    if (dtype != FLARE_BF16 || a.MB != 8 || nk) return FLARE_ERR_UNSUPPORTED;
    if (qtype == FLARE_BF16)
      return D == 16 ? launch_decode_k<bf16, bf16, 16, false, false, false, 8, true>(a, lds, st)
                     : launch_decode_k<bf16, bf16, 32, false, false, false, 8, true>(a, lds, st);
    return D == 16 ? launch_decode_k<bf16, float, 16, false, false, false, 8, true>(a, lds, st)
                   : launch_decode_k<bf16, float, 32, false, false, false, 8, true>(a, lds, st);
  }
  if (dtype == FLARE_BF16) {
    if (qtype == FLARE_BF16)
      return D == 16 ? launch_decode_t<bf16, bf16, 16>(a, lds, nk, st) : launch_decode_t<bf16, bf16, 32>(a, lds, nk, st);
    return D == 16 ? launch_decode_t<bf16, float, 16>(a, lds, nk, st) : launch_decode_t<bf16, float, 32>(a, lds, nk, st);
  }
  if (qtype != FLARE_F32 || nm.qmul1) return FLARE_ERR_UNSUPPORTED;
  return D == 16 ? launch_decode_t<float, float, 16>(a, lds, nk, st) : launch_decode_t<float, float, 32>(a, lds, nk, st);
}

float pick_scale(float scale, int D) { return scale > 0.f ? scale : 1.0f / sqrtf((float)D); }

// Workspace carve-up: the encode's split partials, then float32 buffers the
// call needs internally.
struct WsLayout {
  size_t part_acc = 0, part_al = 0, z = 0, l = 0, q = 0, k = 0, total = 0;
  size_t km = 0, kh = 0;  // per-split and per-head key-norm maxima (bf16 forwards with a decode)
  bool kmax = false;
};

WsLayout ws_layout(const Dev& dev, int op, int B, int H, int N, int M, int D, int dtype, bool need_z, bool need_q) {
  WsLayout w;
  const int BH = B * H;
  size_t off = 0;
  if (op != FLARE_OP_DECODE && N > 0) {
    // the split partials of one encode over all heads
    const EncPlan p = plan_encode(dev, BH, N, M, dtype);
    const size_t acc = align256((size_t)BH * p.pmax * M * D * sizeof(float));
    const size_t al = align256((size_t)BH * p.pmax * M * sizeof(float2));
    w.part_acc = 0;
    w.part_al = acc;
    off = acc + al;
    if (dtype == FLARE_BF16 && op != FLARE_OP_ENCODE) {  // the encode's key norms, for the decode
      w.kmax = true;
      w.km = off; off += align256((size_t)BH * p.pmax * sizeof(float));
      w.kh = off; off += align256((size_t)BH * sizeof(float));
    }
  }
  if (need_z) { w.z = off; off += align256((size_t)BH * M * D * sizeof(float)); w.l = off; off += align256((size_t)BH * M * sizeof(float)); }
  if (need_q) { w.q = off; off += align256((size_t)BH * M * D * sizeof(float)); }
  if (op == FLARE_OP_FORWARD_PROJ || op == FLARE_OP_PP_FORWARD_PROJ) {  // the projected keys, bf16 [B,H,N,D]
    w.k = off;
    off += align256((size_t)BH * N * D * 2);
  }
  w.total = off;
  return w;
}

// The one-workgroup-per-head forward (head_kernel) serves bf16, D = 32 and
// M = 64 or 128 without normalisations, when the heads alone occupy at least
// half of the compute units and each is short: there the split of a head
// across workgroups gains less than the kernel boundaries cost.  Up to
// kHeadMaxN tokens for FLARE++ (five launches saved), and for FLARE (three)
// half of that unless the heads fill every compute unit.  (For
// FLARE++, two workgroups per head, both encoding all of its tokens and each
// decoding half, were no faster at a quarter to half of the compute units:
// the doubled key and value reads slowed both encodes by what the halved
// decode saved.)
constexpr int kHeadMaxN = 8192;

// The FLARE++ encodes by (head, latent block) with a separate decode
// (latent_kernel) serve the inputs of head_kernel (bf16, D = 32, no
// normalisations) for M a multiple of 32 and 2048 to kHeadMaxN tokens per
// head, when the B H M / 32 workgroups fill more than half of the compute
// units and at most all of them.  Each head's keys and values are then read
// by M / 32 workgroups, so the encodes gain less than the spread suggests:
// at the long-sequence workload 58.5-58.9 against 61.8-62.4 us for
// head_kernel.  For FLARE, with one encode, it was no faster than head_kernel
// or the launch sequence, and for shorter heads the second launch costs more
// than the spread gains.
bool latent_applies(const Dev& dev, int BH, int N, int M, int D, int dtype, const WsLayout& w) {
  if (dtype != FLARE_BF16 || D != 32 || (M & 31) || N < 2048 || N > kHeadMaxN || !w.kmax) return false;
  const long long wgs = (long long)BH * (M / 32);
  if (2 * wgs <= dev.cus || wgs > dev.cus) return false;
  return kLatLds + 1024 <= dev.lds_max && decode_lds(dtype, D, M) <= dev.lds_max;
}

bool head_applies(const Dev& dev, bool pp, int BH, int N, int M, int D, int dtype, const WsLayout& w) {
  if (dtype != FLARE_BF16 || D != 32 || (M != 64 && M != 128)) return false;
  const int nmax = pp || BH >= dev.cus ? kHeadMaxN : kHeadMaxN / 2;
  if (N < 1 || N > nmax || 2 * (long long)BH < dev.cus || !w.kmax) return false;
  return (M == 64 ? head_lds<2>() : head_lds<4>()) + 1024 <= dev.lds_max;
}

template <int MB, bool PP>
int launch_head(const HeadArgs& a, int BH, hipStream_t st) {
  static_assert(head_tile_bytes<MB>() >= (size_t)(MB * 32 * (32 + 8) + 32 * (MB * 32 + 4)) * sizeof(bf16),
                "the decode's staging fits in the encode's tiles");
  const size_t lds = head_lds<MB>();
  if (lds > 65536 && hipFuncSetAttribute((const void*)head_kernel<MB, PP>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return FLARE_ERR_HIP;
  return launch(head_kernel<MB, PP>, dim3(BH), dim3(kHeadWaves * 64), lds, st, a);
}

// The plan of one piece per head (its WN splits the token lanes), and the
// routing encode and decode arguments: queries Q (bf16 with q_batched, or the
// float32 blended ones), kh: [B H] floats of workspace for the heads' largest
// squared routing-key norms.
HeadArgs head_args(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z, float* L, int B,
                   int H, int N, int M, float qs, float* kh, EncPlan& p) {
  const int BH = B * H;
  p = EncPlan{};
  p.G = M / 32;
  p.WN = kHeadWaves / p.G;
  p.nwg = BH;  // piece i is head i
  p.total = (long long)BH * N;
  p.pmax = p.WN;
  HeadArgs a{};
  a.re = encode_args(Q, q_batched, K, V, 0, H, N, M, qs, nullptr, nullptr, p, Norms{}, kh);
  a.d = DecArgs{};
  a.d.Q = Q; a.d.K = K; a.d.Z = Z; a.d.Y = Y; a.d.kmax = kh;
  a.d.total = p.total;
  a.d.q_batched = q_batched; a.d.H = H; a.d.N = N; a.d.M = M; a.d.MB = M / 32; a.d.nwg = BH; a.d.bh0 = 0;
  a.d.qscale = qs;
  a.Z = Z; a.L = L; a.H = H;
  return a;
}

// The FLARE++ encodes by (head, latent block) followed by the decode: Qb, Z,
// L and Y as the launch sequence writes them; kh: [B H] floats of workspace.
int launch_latent(const Dev& dev, const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                  const void* K, const void* V, void* Y, float* Qb, float* Z, float* L, int B, int H, int N, int M,
                  float qs, float* kh, hipStream_t st) {
  const int BH = B * H, D = 32;
  EncPlan p{};
  p.G = 1;
  p.WN = kHeadWaves;
  p.nwg = BH;  // piece i is head i
  p.total = (long long)BH * N;
  p.pmax = p.WN;
  HeadArgs a{};
  a.se = encode_args(Qs, 0, Ks, Vs, 0, H, N, M, qs, nullptr, nullptr, p, Norms{}, nullptr);
  a.re = encode_args(Qb, 1, K, V, 0, H, N, M, qs, nullptr, nullptr, p, Norms{}, kh);
  a.Qf = (const bf16*)Qf; a.gate = gate; a.Qout = Qb;
  a.Z = Z; a.L = L; a.H = H; a.nbh = BH;
  if (kLatLds > 65536 && hipFuncSetAttribute((const void*)latent_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kLatLds) != hipSuccess)
    return FLARE_ERR_HIP;
  const int rc = launch(latent_kernel, dim3(BH * (M / 32)), dim3(kHeadWaves * 64), kLatLds, st, a);
  if (rc) return rc;
  return launch_decode(dev, Qb, FLARE_F32, 1, K, Z, Y, 0, BH, H, N, M, D, FLARE_BF16, qs, Norms{}, st, kh);
}

// FLARE forward of B H heads of N tokens with bf16 queries (head_applies
// holds): Z, L and Y as the launch sequence writes them.
int launch_flare_head(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z, float* L, int B,
                      int H, int N, int M, float qs, float* kh, hipStream_t st) {
  EncPlan p;
  const HeadArgs a = head_args(Q, q_batched, K, V, Y, Z, L, B, H, N, M, qs, kh, p);
  return M == 64 ? launch_head<2, false>(a, B * H, st) : launch_head<4, false>(a, B * H, st);
}

// FLARE++ forward (head_applies holds, no normalisations): Qb, Z, L and Y as
// the launch sequence writes them.
int launch_pp_head(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate, const void* K,
                   const void* V, void* Y, float* Qb, float* Z, float* L, int B, int H, int N, int M, float qs,
                   float* kh, hipStream_t st) {
  EncPlan p;
  HeadArgs a = head_args(Qb, 1, K, V, Y, Z, L, B, H, N, M, qs, kh, p);
  a.se = encode_args(Qs, 0, Ks, Vs, 0, H, N, M, qs, nullptr, nullptr, p, Norms{}, nullptr);
  a.Qf = (const bf16*)Qf; a.gate = gate; a.Qout = Qb;
  return M == 64 ? launch_head<2, true>(a, B * H, st) : launch_head<4, true>(a, B * H, st);
}

}  // namespace

#include "backward.h"
#include "proj.h"

// ----------------------------------------------------------------------------
// Scratch of the allocation-free entry point: a file-scope device array, one
// copy per GPU, resolved to a device address once per device.  Host code
// never uses the array's name as an address (on the host it is a stand-in,
// not device memory); kernels get the resolved pointer.
// ----------------------------------------------------------------------------
constexpr size_t kScratchBytes = FLARE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// Device address of the current device's scratch array.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLARE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FLARE_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return FLARE_OK;
}
}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------
extern "C" {

const char* flare_status_string(int status) {
  switch (status) {
    case FLARE_OK: return "ok";
    case FLARE_ERR_INVALID_ARG: return "invalid argument";
    case FLARE_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case FLARE_ERR_WORKSPACE: return "workspace too small";
    case FLARE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t flare_workspace_size(int op, int B, int H, int N, int M, int D, int dtype) {
  if (check_common(B, H, N, M, D, dtype, 0) != FLARE_OK) return 0;
  if (op < FLARE_OP_ENCODE || op > FLARE_OP_PP_FORWARD_PROJ) return 0;
  if (op == FLARE_OP_DECODE) return 0;
  Dev dev;
  if (query_dev(dev) != FLARE_OK) return 0;
  if (op == FLARE_OP_BACKWARD || op == FLARE_OP_ENCODE_BACKWARD || op == FLARE_OP_PP_BACKWARD ||
      op == FLARE_OP_PP_BACKWARD_NORM) {
    if (dtype == FLARE_F32) {
      if (op == FLARE_OP_PP_BACKWARD_NORM) return 0;
      if (op == FLARE_OP_PP_BACKWARD) return pp_bwd32_layout(dev, B, H, N, M, D).total;
      return bwd32_layout(dev, op == FLARE_OP_BACKWARD, B, H, N, M, D).total;
    }
    if (op == FLARE_OP_PP_BACKWARD) return pp_bwd_layout(dev, B, H, N, M, D).total;
    if (op == FLARE_OP_PP_BACKWARD_NORM) return pp_bwd_norm_layout(dev, B, H, N, M, D).total;
    return bwd_layout(dev, op == FLARE_OP_BACKWARD, B, H, N, M, D).total;
  }
  if (op == FLARE_OP_FORWARD_PROJ || op == FLARE_OP_PP_FORWARD_PROJ) {
    if (dtype != FLARE_BF16 || D != 32) return 0;
  }
  const bool need_z = op == FLARE_OP_FORWARD || op == FLARE_OP_PP_FORWARD || op == FLARE_OP_FORWARD_PROJ ||
                      op == FLARE_OP_PP_FORWARD_PROJ;
  const bool need_q = op == FLARE_OP_PP_FORWARD || op == FLARE_OP_PP_FORWARD_PROJ;
  return ws_layout(dev, op, B, H, N, M, D, dtype, need_z, need_q).total;
}

int flare_encode(const void* Q, int q_batched, const void* K, const void* V, float* Z, float* L, int B, int H,
                 int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, q_batched);
  if (rc) return rc;
  if (!Q || !Z || (N > 0 && (!K || !V))) return FLARE_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Z) || !aligned16(ws)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  const WsLayout w = ws_layout(dev, FLARE_OP_ENCODE, B, H, N, M, D, dtype, false, false);
  if (ws_bytes < w.total || (w.total > 0 && !ws)) return FLARE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const float qs = pick_scale(scale, D) * kLog2e;
  const int BH = B * H;
  const EncPlan p = plan_encode(dev, BH, N, M, dtype);
  float* pacc = (float*)((char*)ws + w.part_acc);
  float2* pal = (float2*)((char*)ws + w.part_al);
  if (N > 0) {
    rc = launch_encode(Q, dtype, q_batched, K, V, 0, H, N, M, D, dtype, qs, pacc, pal, p, Norms{}, st);
    if (rc) return rc;
  }
  return launch_merge(p, pacc, pal, 0, BH, H, N, M, D, Z, L, nullptr, FLARE_F32, nullptr, nullptr, 0, nullptr, 0.f,
                      st);
}

int flare_decode(const void* Q, int q_batched, const void* K, const float* Z, void* Y, int B, int H, int N, int M,
                 int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  int rc = check_common(B, H, N, M, D, dtype, q_batched);
  if (rc) return rc;
  if (!Q || !Z || (N > 0 && (!K || !Y))) return FLARE_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Z) || !aligned16(Y)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (decode_lds(dtype, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const float qs = pick_scale(scale, D) * kLog2e;
  return launch_decode(dev, Q, dtype, q_batched, K, Z, Y, 0, B * H, H, N, M, D, dtype, qs, Norms{},
                       (hipStream_t)stream);
}

// Shared by flare_forward and the routing half of flare_pp_forward: encode ->
// merge -> decode over all heads.  Q has element type qtype; nm carries the
// routing keys' normalisation (N_0 rows, and their scale moved onto Q).
static int routing(const Dev& dev, const void* Q, int qtype, int q_batched, const void* K, const void* V, void* Y,
                   float* Z, float* L, int B, int H, int N, int M, int D, int dtype, float qs, char* ws,
                   const WsLayout& w, const Norms& nm, hipStream_t st) {
  const int BH = B * H;
  float* pacc = (float*)(ws + w.part_acc);
  float2* pal = (float2*)(ws + w.part_al);
  const EncPlan p = plan_encode(dev, BH, N, M, dtype);
  float* km = w.kmax ? (float*)(ws + w.km) : nullptr;
  float* kh = w.kmax ? (float*)(ws + w.kh) : nullptr;
  const bool no_norms = !nm.norm_q && !nm.qmul0 && !nm.qmul1 && !nm.norm_k;
  if (qtype == FLARE_BF16 && no_norms && head_applies(dev, false, BH, N, M, D, dtype, w))  // many short heads
    return launch_flare_head(Q, q_batched, K, V, Y, Z, L, B, H, N, M, qs, kh, st);
  int rc;
  if (N > 0) {
    rc = launch_encode(Q, qtype, q_batched, K, V, 0, H, N, M, D, dtype, qs, pacc, pal, p, nm, st, km);
    if (rc) return rc;
  }
  if (decode_merges(p, BH, N, M, dtype, nm)) {  // the decode merges the splits as it stages Z
    DecMerge mg;
    mg.p = &p; mg.part_acc = pacc; mg.part_al = pal; mg.part_km = km; mg.Z = Z; mg.L = L;
    return launch_decode(dev, Q, qtype, q_batched, K, Z, Y, 0, BH, H, N, M, D, dtype, qs, nm, st, nullptr, &mg);
  }
  rc = launch_merge(p, pacc, pal, 0, BH, H, N, M, D, Z, L, nullptr, FLARE_F32, nullptr, nullptr, 0, nullptr, 0.f, st,
                    km, kh);
  if (rc) return rc;
  return launch_decode(dev, Q, qtype, q_batched, K, Z, Y, 0, BH, H, N, M, D, dtype, qs, nm, st, kh);
}

// flare_forward with the workspace at ws (ws_bytes long), or, when ws_bytes
// is 0 and scratch is set, in the file-scope scratch array of the current
// device (checked against its size before anything is enqueued).
static int forward_impl(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z_out,
                        float* L_out, int B, int H, int N, int M, int D, int dtype, float scale, void* ws,
                        size_t ws_bytes, bool scratch, void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, q_batched);
  if (rc) return rc;
  if (!Q || (N > 0 && (!K || !V || !Y))) return FLARE_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Y) || !aligned16(Z_out) ||
      !aligned16(L_out) || !aligned16(ws))
    return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (decode_lds(dtype, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(dev, FLARE_OP_FORWARD, B, H, N, M, D, dtype, true, false);
  if (scratch) {
    if (w.total > kScratchBytes) return FLARE_ERR_WORKSPACE;
    if ((rc = scratch_address(&ws))) return rc;
    ws_bytes = kScratchBytes;
  }
  if (ws_bytes < w.total || (w.total > 0 && !ws)) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  float* Z = Z_out ? Z_out : (float*)(wsc + w.z);
  float* L = L_out ? L_out : (float*)(wsc + w.l);
  const float qs = pick_scale(scale, D) * kLog2e;
  return routing(dev, Q, dtype, q_batched, K, V, Y, Z, L, B, H, N, M, D, dtype, qs, wsc, w, Norms{},
                 (hipStream_t)stream);
}

int flare_forward(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z_out, float* L_out,
                  int B, int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                  void* stream) {
  return forward_impl(Q, q_batched, K, V, Y, Z_out, L_out, B, H, N, M, D, dtype, scale, ws, ws_bytes, false,
                      stream);
}

int flare_forward_noalloc(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z_out,
                          float* L_out, int B, int H, int N, int M, int D, int dtype, float scale, void* stream) {
  return forward_impl(Q, q_batched, K, V, Y, Z_out, L_out, B, H, N, M, D, dtype, scale, nullptr, 0, true, stream);
}

int flare_pp_forward_norm(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                          const void* K, const void* V, void* Y, float* Q_out, float* Z_out, float* L_out, int B,
                          int H, int N, int M, int D, int dtype, float scale, int norm_flags, const float* alpha_qs,
                          const float* alpha_ks, const float* alpha_k, float eps, void* ws, size_t ws_bytes,
                          void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, 0);
  if (rc) return rc;
  if (!Qs || !Qf || !gate || (N > 0 && (!Ks || !Vs || !K || !V || !Y))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {Qs, Ks, Vs, Qf, gate, K, V, Y, Q_out, Z_out, L_out, ws, alpha_qs, alpha_ks, alpha_k};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  if (norm_flags & ~FLARE_NORM_ALL) return FLARE_ERR_INVALID_ARG;
  if (norm_flags && !(eps > 0.f)) return FLARE_ERR_INVALID_ARG;
  if (norm_flags && dtype != FLARE_BF16) return FLARE_ERR_UNSUPPORTED;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (decode_lds(dtype, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(dev, FLARE_OP_PP_FORWARD, B, H, N, M, D, dtype, true, true);
  if (ws_bytes < w.total || (w.total > 0 && !ws)) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  float* Qb = Q_out ? Q_out : (float*)(wsc + w.q);
  float* Z = Z_out ? Z_out : (float*)(wsc + w.z);
  float* L = L_out ? L_out : (float*)(wsc + w.l);
  const float qs = pick_scale(scale, D) * kLog2e;
  const int BH = B * H;
  // Synthesis: seeds N_a (N_0 rows, then alpha_qs), keys N_0 rows with their
  // scale alpha_ks moved onto the seeds, and, when the values are the keys,
  // onto the merged latents too (they are linear in the values).
  const bool nks = norm_flags & FLARE_NORM_KS;
  Norms syn;
  syn.norm_q = (norm_flags & FLARE_NORM_QS) ? 1 : 0;
  syn.qmul0 = syn.norm_q ? alpha_qs : nullptr;
  syn.qmul1 = nks ? alpha_ks : nullptr;
  syn.norm_k = nks;
  syn.eps = eps;
  const float* zmul = (nks && Ks == Vs) ? alpha_ks : nullptr;
  // Routing: keys N_0 rows with their scale alpha_k moved onto the queries.
  Norms rt;
  rt.norm_k = norm_flags & FLARE_NORM_K;
  rt.qmul1 = rt.norm_k ? alpha_k : nullptr;
  rt.eps = eps;
  if (!norm_flags) {  // many short heads: one workgroup per latent block, or per head
    if (latent_applies(dev, BH, N, M, D, dtype, w))
      return launch_latent(dev, Qs, Ks, Vs, Qf, gate, K, V, Y, Qb, Z, L, B, H, N, M, qs, (float*)(wsc + w.kh), st);
    if (head_applies(dev, true, BH, N, M, D, dtype, w))
      return launch_pp_head(Qs, Ks, Vs, Qf, gate, K, V, Y, Qb, Z, L, B, H, N, M, qs, (float*)(wsc + w.kh), st);
  }
  const EncPlan p = plan_encode(dev, BH, N, M, dtype);
  // Synthesis encode over all heads, merged straight into the blended queries.
  float* pacc = (float*)(wsc + w.part_acc);
  float2* pal = (float2*)(wsc + w.part_al);
  if (N > 0) {
    rc = launch_encode(Qs, dtype, 0, Ks, Vs, 0, H, N, M, D, dtype, qs, pacc, pal, p, syn, st);
    if (rc) return rc;
  }
  rc = launch_merge(p, pacc, pal, 0, BH, H, N, M, D, nullptr, nullptr, Qf, dtype, gate, Qb,
                    (norm_flags & FLARE_NORM_QF) ? 1 : 0, zmul, eps, st);
  if (rc) return rc;
  // Routing with the per-batch float32 queries.
  return routing(dev, Qb, FLARE_F32, 1, K, V, Y, Z, L, B, H, N, M, D, dtype, qs, wsc, w, rt, st);
}

// Routing from the block input: the encode projects K and V per tile and
// writes the keys to Kbuf, the merge forms Z and L, the decode reads Kbuf.
static int routing_proj(const Dev& dev, const void* X, const void* WK, const void* WV, bf16* Kbuf, const void* Q,
                        int qtype, int q_batched, void* Y, float* Z, float* L, int B, int H, int N, int M, int D,
                        float qs, char* ws, const WsLayout& w, const Norms& nm, hipStream_t st) {
  const int BH = B * H;
  float* pacc = (float*)(ws + w.part_acc);
  float2* pal = (float2*)(ws + w.part_al);
  const EncPlan p = plan_encode(dev, BH, N, M, FLARE_BF16);
  float* km = w.kmax ? (float*)(ws + w.km) : nullptr;
  float* kh = w.kmax ? (float*)(ws + w.kh) : nullptr;
  int rc;
  if (N > 0) {
    rc = launch_encode_proj(X, WK, WV, Kbuf, Q, qtype, q_batched, H, N, M, qs, pacc, pal, p, nm, st, km);
    if (rc) return rc;
  }
  rc = launch_merge(p, pacc, pal, 0, BH, H, N, M, D, Z, L, nullptr, FLARE_F32, nullptr, nullptr, 0, nullptr, 0.f, st,
                    km, kh);
  if (rc) return rc;
  // the keys in Kbuf are already normalised: the decode only moves their scale onto the queries
  Norms dn;
  dn.qmul1 = nm.qmul1;
  return launch_decode(dev, Q, qtype, q_batched, Kbuf, Z, Y, 0, BH, H, N, M, D, FLARE_BF16, qs, dn, st, kh);
}

static int check_proj(int B, int H, int N, int M, int D, int C, int dtype) {
  int rc = check_common(B, H, N, M, D, dtype, 0);
  if (rc) return rc;
  if (dtype != FLARE_BF16 || D != 32 || C != kProjC) return FLARE_ERR_UNSUPPORTED;
  if ((long long)B * N * C >= (1LL << 31)) return FLARE_ERR_UNSUPPORTED;
  return FLARE_OK;
}

int flare_forward_proj(const void* X, const void* WK, const void* WV, const void* Q, int q_batched, void* Y,
                       void* K_out, float* Z_out, float* L_out, int B, int H, int N, int M, int D, int C, int dtype,
                       float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_proj(B, H, N, M, D, C, dtype);
  if (rc) return rc;
  if (q_batched != 0 && q_batched != 1) return FLARE_ERR_INVALID_ARG;
  if (!Q || !WK || !WV || (N > 0 && (!X || !Y))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {X, WK, WV, Q, Y, K_out, Z_out, L_out, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (decode_lds(dtype, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(dev, FLARE_OP_FORWARD_PROJ, B, H, N, M, D, dtype, true, false);
  if (ws_bytes < w.total || (w.total > 0 && !ws)) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  float* Z = Z_out ? Z_out : (float*)(wsc + w.z);
  float* L = L_out ? L_out : (float*)(wsc + w.l);
  bf16* Kb = K_out ? (bf16*)K_out : (bf16*)(wsc + w.k);
  const float qs = pick_scale(scale, D) * kLog2e;
  return routing_proj(dev, X, WK, WV, Kb, Q, FLARE_BF16, q_batched, Y, Z, L, B, H, N, M, D, qs, wsc, w, Norms{},
                      (hipStream_t)stream);
}

int flare_pp_forward_proj(const void* X, const void* WKs, const void* WK, const void* WV, const void* Qs,
                          const void* Qf, const float* gate, void* Y, float* Q_out, void* K_out, float* Z_out,
                          float* L_out, int B, int H, int N, int M, int D, int C, int dtype, float scale,
                          int norm_flags, const float* alpha_qs, const float* alpha_k, float eps, void* ws,
                          size_t ws_bytes, void* stream) {
  int rc = check_proj(B, H, N, M, D, C, dtype);
  if (rc) return rc;
  if (!Qs || !Qf || !gate || !WKs || !WK || !WV || (N > 0 && (!X || !Y))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {X, WKs, WK, WV, Qs, Qf, gate, Y, Q_out, K_out, Z_out, L_out, ws, alpha_qs, alpha_k};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  if (norm_flags & ~FLARE_NORM_ALL) return FLARE_ERR_INVALID_ARG;
  if (norm_flags && !(eps > 0.f)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (decode_lds(dtype, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(dev, FLARE_OP_PP_FORWARD_PROJ, B, H, N, M, D, dtype, true, true);
  if (ws_bytes < w.total || (w.total > 0 && !ws)) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  float* Qb = Q_out ? Q_out : (float*)(wsc + w.q);
  float* Z = Z_out ? Z_out : (float*)(wsc + w.z);
  float* L = L_out ? L_out : (float*)(wsc + w.l);
  bf16* Kb = K_out ? (bf16*)K_out : (bf16*)(wsc + w.k);
  const float qs = pick_scale(scale, D) * kLog2e;
  const int BH = B * H;
  // Synthesis from X W~_K, the values being the (normalised) keys (App. A.6).
  Norms syn;
  syn.norm_q = (norm_flags & FLARE_NORM_QS) ? 1 : 0;
  syn.qmul0 = syn.norm_q ? alpha_qs : nullptr;
  syn.norm_k = norm_flags & FLARE_NORM_KS;
  syn.eps = eps;
  const EncPlan p = plan_encode(dev, BH, N, M, dtype);
  float* pacc = (float*)(wsc + w.part_acc);
  float2* pal = (float2*)(wsc + w.part_al);
  if (N > 0) {
    rc = launch_encode_proj(X, WKs, WKs, nullptr, Qs, FLARE_BF16, 0, H, N, M, qs, pacc, pal, p, syn, st);
    if (rc) return rc;
  }
  rc = launch_merge(p, pacc, pal, 0, BH, H, N, M, D, nullptr, nullptr, Qf, FLARE_BF16, gate, Qb,
                    (norm_flags & FLARE_NORM_QF) ? 1 : 0, nullptr, eps, st);
  if (rc) return rc;
  // Routing from X W_K (N_0 rows, the scale alpha_k moved onto the queries) and X W_V.
  Norms rt;
  rt.norm_k = norm_flags & FLARE_NORM_K;
  rt.qmul1 = rt.norm_k ? alpha_k : nullptr;
  rt.eps = eps;
  return routing_proj(dev, X, WK, WV, Kb, Qb, FLARE_F32, 1, Y, Z, L, B, H, N, M, D, qs, wsc, w, rt, st);
}

int flare_pp_forward(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                     const void* K, const void* V, void* Y, float* Q_out, float* Z_out, float* L_out, int B, int H,
                     int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream) {
  return flare_pp_forward_norm(Qs, Ks, Vs, Qf, gate, K, V, Y, Q_out, Z_out, L_out, B, H, N, M, D, dtype, scale, 0,
                               nullptr, nullptr, nullptr, 0.f, ws, ws_bytes, stream);
}

}  // extern "C"
