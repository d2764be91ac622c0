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
// Kernels (all 256 threads = 4 waves of 64):
//   encode_kernel  -- split-N encode partials.  The flattened (head, token)
//                     range of a launch is cut into one contiguous piece per
//                     workgroup; token tiles of 128 are staged in LDS (K
//                     row-major, V transposed) and each wave owns up to 64
//                     latents.  Scores S^T = K Q^T and the latent update
//                     Z^T += V^T P^T run on 32x32 MFMA tiles; one lane owns
//                     one latent column, so the softmax statistics over the
//                     tokens are in-lane plus one permlane32 swap.  A split
//                     emits the running (shift, sum, accumulator) triple.
//   merge_kernel   -- log-sum-exp merge of the splits in a fixed order
//                     (Sec. 3.3, App. B.3); optionally the FLARE++ blend.
//   decode_kernel  -- per-token softmax over the latents: the scaled queries
//                     and the latents stay in LDS for a head, every wave takes
//                     64 tokens, S = Q K^T and Y^T += Z^T P run on MFMA with
//                     one lane per token column.
// Scores are kept in log2 units: the queries are pre-multiplied by
// s*log2(e) so every exponential is a single v_exp_f32.  The running shift
// enters the score MFMA as its accumulator input, and it is only raised when
// a tile's maximum exceeds it by more than kTheta (otherwise the stale shift
// keeps every exponential below 2^kTheta), so the common tile costs one
// exp, one add and one convert per score.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "flare.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;      // 4 waves per workgroup
constexpr int kTile = 128;         // tokens per encode LDS tile (4 blocks of 32)
constexpr int kDecGroup = 256;     // tokens per decode step of a workgroup (64 per wave)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTheta = 8.0f;     // lazy-rescale threshold, log2 units

// ----------------------------------------------------------------------------
// Small device helpers
// ----------------------------------------------------------------------------
template <typename T> __device__ inline float to_f(T x) { return (float)x; }
template <typename T> __device__ inline T from_f(float x) { return (T)x; }  // RNE for bf16

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

// Flattened (head, token) range of workgroup i when `total` tokens are cut
// into `nwg` contiguous pieces.
__host__ __device__ inline long long piece_start(long long i, long long total, int nwg) {
  return i * total / nwg;
}
__host__ __device__ inline int piece_of(long long x, long long total, int nwg) {
  long long i = x * nwg / total;
  if (i >= nwg) i = nwg - 1;
  while (i + 1 < nwg && piece_start(i + 1, total, nwg) <= x) ++i;
  while (i > 0 && piece_start(i, total, nwg) > x) --i;
  return (int)i;
}

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

template <int D> __device__ inline f32x16 qk_mma(const QKOp<bf16, D>& a, const QKOp<bf16, D>& b, f32x16 c) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v[st], b.v[st], c, 0, 0, 0);
  return c;
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

// acc += X^T P, P being the (already exponentiated) score tile in registers.
__device__ inline f32x16 pv_mma(const PVOp<bf16>& a, const f32x16& p, f32x16 acc) {
  bf16x8 b0, b1;
#pragma unroll
  for (int s = 0; s < 8; ++s) { b0[s] = (bf16)p[s]; b1[s] = (bf16)p[8 + s]; }
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a0, b0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.a1, b1, acc, 0, 0, 0);
  return acc;
}
__device__ inline f32x16 pv_mma(const PVOp<float>& a, const f32x16& p, f32x16 acc) {
#pragma unroll
  for (int j = 0; j < 16; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[j], p[j], acc, 0, 0, 0);
  return acc;
}

// One online-softmax step on a 32x32 score tile whose column (this lane's
// latent in the encode, token in the decode) is the softmax row.  On entry
// s = raw score - shift (the shift entered as -shift through the MFMA
// accumulator `negshift`); on exit s holds the weights exp2(s).  The shift is
// raised to the tile maximum when that exceeds it by more than kTheta, or on
// the first non-empty tile; the running sum and accumulator are rescaled then.
__device__ inline void online_step(f32x16& s, f32x16& negshift, bool& started, float& lsum, f32x16& acc) {
  float t = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) t = fmaxf(t, s[r]);
  t = pair_max(t);
  const bool need = (t > kTheta) || (!started && t > -INFINITY);
  if (need) {
    const float f = started ? fast_exp2(-t) : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s[r] -= t; negshift[r] -= t; acc[r] *= f; }
    lsum *= f;
    started = true;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) { s[r] = fast_exp2(s[r]); lsum += s[r]; }
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
  long long total;    // nbh * N
  int q_batched, v_alias, H, N, M, G, nwg, pmax, bh0;
  float qscale;       // s * log2(e)
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
        else zero_pv(vop);
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
          acc[mb] = pv_mma(vop, s, acc[mb]);
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
      const float ltot = pair_sum(lsum[mb]);
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
  long long total;
  int N, M, D, H, WN, nwg, pmax, bh0, nbh;
};

template <typename QT>
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeArgs a) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)a.nbh * a.M * a.D) return;
  const int d = (int)(idx % a.D);
  const long long t = idx / a.D;
  const int m = (int)(t % a.M);
  const int bhl = (int)(t / a.M);
  const int bh = a.bh0 + bhl;
  float z = 0.f, lse = -INFINITY;
  if (a.N > 0) {
    const long long hb = (long long)bhl * a.N;
    const int w0 = piece_of(hb, a.total, a.nwg);
    const int w1 = piece_of(hb + a.N - 1, a.total, a.nwg);
    const int cnt = (w1 - w0 + 1) * a.WN;
    const size_t base = (size_t)bhl * a.pmax;
    float A = -INFINITY;
    for (int p = 0; p < cnt; ++p) {
      const float2 v = a.part_al[(base + p) * a.M + m];
      if (v.y > 0.f) A = fmaxf(A, v.x);
    }
    if (A > -INFINITY) {
      float den = 0.f, num = 0.f;
      for (int p = 0; p < cnt; ++p) {
        const float2 v = a.part_al[(base + p) * a.M + m];
        if (v.y > 0.f) {
          const float w = fast_exp2(v.x - A);
          den += w * v.y;
          num += w * a.part_acc[((base + p) * a.M + m) * a.D + d];
        }
      }
      z = num / den;
      lse = kLn2 * (A + __builtin_amdgcn_logf(den));
    }
  }
  const size_t o = ((size_t)bh * a.M + m) * a.D + d;
  if (a.Qout) {
    const int h = bh % a.H;
    const float qf = to_f(reinterpret_cast<const QT*>(a.Qf)[((size_t)h * a.M + m) * a.D + d]);
    a.Qout[o] = qf + a.gate[h] * z;
  } else {
    a.Z[o] = z;
    if (a.L && d == 0) a.L[(size_t)bh * a.M + m] = lse;
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
};

template <typename T, int D> struct DecLds {
  static constexpr int E = 16 / sizeof(T);
  static constexpr int QST = D + E;
  __host__ __device__ static size_t zst(int MB) { return (size_t)MB * 32 + (sizeof(T) == 2 ? 8 : 4); }
  static size_t bytes(int MB) { return ((size_t)MB * 32 * QST + (size_t)D * zst(MB)) * sizeof(T); }
};

template <typename T, typename QT, int D>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecArgs a) {
  using L = DecLds<T, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int MB = a.MB, Mp = 32 * MB, M = a.M, N = a.N;
  T* qs = reinterpret_cast<T*>(smem);
  T* zt = qs + (size_t)Mp * L::QST;
  const int zst = (int)L::zst(MB);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, g = lane >> 5;
  const bool mask_tail = (M & 31) != 0;

  long long x = piece_start(blockIdx.x, a.total, a.nwg);
  const long long xe = piece_start(blockIdx.x + 1, a.total, a.nwg);
  while (x < xe) {
    const int bhl = (int)(x / N);
    const long long hb = (long long)bhl * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int bh = a.bh0 + bhl;
    const int h = bh % a.H;

    // Stage this head's scaled queries (rows = latents) and transposed latents.
    __syncthreads();
    const QT* Qh = reinterpret_cast<const QT*>(a.Q) + (size_t)(a.q_batched ? bh : h) * M * D;
    const float* Zh = a.Z + (size_t)bh * M * D;
    for (int i = threadIdx.x; i < Mp * D; i += kThreads) {
      const int m = i / D, d = i % D;
      const bool ok = m < M;
      qs[m * L::QST + d] = from_f<T>(ok ? to_f(Qh[i]) * a.qscale : 0.f);
      zt[d * zst + m] = from_f<T>(ok ? Zh[i] : 0.f);
    }
    __syncthreads();

    const T* Kh = reinterpret_cast<const T*>(a.K) + (size_t)bh * N * D;
    T* Yh = reinterpret_cast<T*>(a.Y) + (size_t)bh * N * D;
    for (int t0 = n_lo + 64 * wave; t0 < n_hi; t0 += kDecGroup) {
      QKOp<T, D> kop[2];
      f32x16 negs[2], acc[2];
      float lsum[2];
      bool started[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = t0 + 32 * j + li;
        if (n < n_hi) load_op<D>(kop[j], Kh + (size_t)n * D, g);
        else zero_op<D>(kop[j]);
#pragma unroll
        for (int r = 0; r < 16; ++r) { negs[j][r] = 0.f; acc[j][r] = 0.f; }
        lsum[j] = 0.f;
        started[j] = false;
      }
      for (int mb = 0; mb < MB; ++mb) {
        QKOp<T, D> qop;
        load_op<D>(qop, qs + (mb * 32 + li) * L::QST, g);
        PVOp<T> zop;
        if (li < D) load_pv(zop, zt + li * zst + mb * 32, g);
        else zero_pv(zop);
        const bool tail = mask_tail && mb == MB - 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f32x16 s = qk_mma<D>(qop, kop[j], negs[j]);
          if (tail) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (mb * 32 + acc_row(r, g) >= M) s[r] = -INFINITY;
          }
          online_step(s, negs[j], started[j], lsum[j], acc[j]);
          acc[j] = pv_mma(zop, s, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = t0 + 32 * j + li;
        const float inv = 1.f / pair_sum(lsum[j]);
        if (n < n_hi) {
          T* dst = Yh + (size_t)n * D;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (8 * c + 4 * g < D) {
              if constexpr (sizeof(T) == 2) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[j][4 * c + i] * inv);
                *reinterpret_cast<bf16x4*>(dst + 8 * c + 4 * g) = v;
              } else {
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = acc[j][4 * c + i] * inv;
                *reinterpret_cast<f32x4*>(dst + 8 * c + 4 * g) = v;
              }
            }
          }
        }
      }
    }
    x = hb + n_hi;
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

// Latent blocks of 32: padded to 1, 2, 4 or 8 so that waves split them evenly.
inline int latent_blocks(int M) {
  int mb = (int)cdiv(M, 32);
  int p = 1;
  while (p < mb) p *= 2;
  return p;
}

struct EncPlan {
  int G, MBW, WN, nwg, pmax;
  long long total;
};

// Workgroups per encode launch: enough to fill the chip twice over, but at
// least 128 tokens each.
constexpr int kEncWgPerCu = 2;
constexpr int kDecWgPerCu = 4;

EncPlan plan_encode(const Dev& dev, int nbh, int N, int M) {
  EncPlan p{};
  const int mbp = latent_blocks(M);
  p.MBW = mbp >= 2 ? 2 : 1;
  p.G = mbp / p.MBW;  // 1, 2 or 4 waves across the latents
  p.WN = 4 / p.G;
  p.total = (long long)nbh * N;
  long long want = (long long)dev.cus * kEncWgPerCu;
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

// Heads per fused encode -> merge -> decode round.  With a nonzero budget a
// group's keys and values are meant to stay resident in the last-level cache
// until its decode re-reads the keys; 0 runs all heads in one round.
#ifndef FLARE_HEAD_GROUP_MB
#define FLARE_HEAD_GROUP_MB 0
#endif
constexpr size_t kHeadGroupBytes = (size_t)FLARE_HEAD_GROUP_MB << 20;

int heads_per_group(int BH, int N, int D, int dtype) {
  const size_t per = (size_t)N * D * (dtype == FLARE_BF16 ? 2 : 4) * 2;
  if (kHeadGroupBytes == 0 || per == 0) return BH;
  size_t g = kHeadGroupBytes / per;
  if (g < 1) g = 1;
  if (g > (size_t)BH) g = BH;
  return (int)g;
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

template <typename T, typename QT, int D, int MBW>
int launch_encode_t(const EncArgs& a, hipStream_t st) {
  const size_t lds = EncLds<T, D>::bytes;
  hipLaunchKernelGGL((encode_kernel<T, QT, D, MBW>), dim3(a.nwg), dim3(kThreads), lds, st, a);
  return hipGetLastError() == hipSuccess ? FLARE_OK : FLARE_ERR_HIP;
}

template <typename T, typename QT>
int launch_encode_d(const EncArgs& a, int D, int MBW, hipStream_t st) {
  if (D == 16) return MBW == 2 ? launch_encode_t<T, QT, 16, 2>(a, st) : launch_encode_t<T, QT, 16, 1>(a, st);
  return MBW == 2 ? launch_encode_t<T, QT, 32, 2>(a, st) : launch_encode_t<T, QT, 32, 1>(a, st);
}

// qtype: element type of Q (FLARE_F32 or FLARE_BF16); dtype: of K and V.
int launch_encode(const Dev& dev, const void* Q, int qtype, int q_batched, const void* K, const void* V, int bh0,
                  int nbh, int H, int N, int M, int D, int dtype, float qscale, float* part_acc, float2* part_al,
                  const EncPlan& p, hipStream_t st) {
  (void)dev;
  EncArgs a;
  a.Q = Q; a.K = K; a.V = V;
  a.part_acc = part_acc; a.part_al = part_al;
  a.total = p.total;
  a.q_batched = q_batched; a.v_alias = (K == V); a.H = H; a.N = N; a.M = M;
  a.G = p.G; a.nwg = p.nwg; a.pmax = p.pmax; a.bh0 = bh0;
  a.qscale = qscale;
  if (dtype == FLARE_BF16) {
    if (qtype == FLARE_BF16) return launch_encode_d<bf16, bf16>(a, D, p.MBW, st);
    return launch_encode_d<bf16, float>(a, D, p.MBW, st);
  }
  if (qtype != FLARE_F32) return FLARE_ERR_UNSUPPORTED;
  return launch_encode_d<float, float>(a, D, p.MBW, st);
}

int launch_merge(const EncPlan& p, const float* part_acc, const float2* part_al, int bh0, int nbh, int H, int N,
                 int M, int D, float* Z, float* L, const void* Qf, int qftype, const float* gate, float* Qout,
                 hipStream_t st) {
  MergeArgs a;
  a.part_acc = part_acc; a.part_al = part_al;
  a.Z = Z; a.L = L; a.Qf = Qf; a.gate = gate; a.Qout = Qout;
  a.total = p.total;
  a.N = N; a.M = M; a.D = D; a.H = H; a.WN = p.WN; a.nwg = p.nwg; a.pmax = p.pmax; a.bh0 = bh0; a.nbh = nbh;
  const long long n = (long long)nbh * M * D;
  const dim3 grid((unsigned)cdiv(n, kThreads));
  if (qftype == FLARE_BF16) hipLaunchKernelGGL((merge_kernel<bf16>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((merge_kernel<float>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? FLARE_OK : FLARE_ERR_HIP;
}

template <typename T, typename QT, int D>
int launch_decode_t(const DecArgs& a, size_t lds, hipStream_t st) {
  if (lds > 65536) {
    if (hipFuncSetAttribute((const void*)decode_kernel<T, QT, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return FLARE_ERR_HIP;
  }
  hipLaunchKernelGGL((decode_kernel<T, QT, D>), dim3(a.nwg), dim3(kThreads), lds, st, a);
  return hipGetLastError() == hipSuccess ? FLARE_OK : FLARE_ERR_HIP;
}

size_t decode_lds(int dtype, int D, int M) {
  const int MB = (int)cdiv(M, 32);
  if (dtype == FLARE_BF16) return D == 16 ? DecLds<bf16, 16>::bytes(MB) : DecLds<bf16, 32>::bytes(MB);
  return D == 16 ? DecLds<float, 16>::bytes(MB) : DecLds<float, 32>::bytes(MB);
}

int launch_decode(const Dev& dev, const void* Q, int qtype, int q_batched, const void* K, const float* Z, void* Y,
                  int bh0, int nbh, int H, int N, int M, int D, int dtype, float qscale, hipStream_t st) {
  if (N == 0) return FLARE_OK;
  DecArgs a;
  a.Q = Q; a.K = K; a.Z = Z; a.Y = Y;
  a.total = (long long)nbh * N;
  a.q_batched = q_batched; a.H = H; a.N = N; a.M = M; a.MB = (int)cdiv(M, 32); a.bh0 = bh0;
  a.qscale = qscale;
  long long want = (long long)dev.cus * kDecWgPerCu;
  long long maxw = cdiv(a.total, 64);
  a.nwg = (int)(want < maxw ? want : maxw);
  const size_t lds = decode_lds(dtype, D, M);
  if (lds > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  if (dtype == FLARE_BF16) {
    if (qtype == FLARE_BF16)
      return D == 16 ? launch_decode_t<bf16, bf16, 16>(a, lds, st) : launch_decode_t<bf16, bf16, 32>(a, lds, st);
    return D == 16 ? launch_decode_t<bf16, float, 16>(a, lds, st) : launch_decode_t<bf16, float, 32>(a, lds, st);
  }
  if (qtype != FLARE_F32) return FLARE_ERR_UNSUPPORTED;
  return D == 16 ? launch_decode_t<float, float, 16>(a, lds, st) : launch_decode_t<float, float, 32>(a, lds, st);
}

float pick_scale(float scale, int D) { return scale > 0.f ? scale : 1.0f / sqrtf((float)D); }

// Workspace carve-up: partials of the largest head group, then float32
// buffers the call needs internally.
struct WsLayout {
  size_t part_acc = 0, part_al = 0, z = 0, l = 0, q = 0, total = 0;
};

WsLayout ws_layout(const Dev& dev, int op, int B, int H, int N, int M, int D, int dtype, bool need_z, bool need_q) {
  WsLayout w;
  const int BH = B * H;
  const int grp = (op == FLARE_OP_ENCODE) ? BH : heads_per_group(BH, N, D, dtype);
  size_t off = 0;
  if (op != FLARE_OP_DECODE && N > 0) {
    // every head-group size that is launched: full groups, the remainder
    // group, and all heads at once for the FLARE++ synthesis encode
    const int groups[3] = {grp, BH % grp ? BH % grp : grp, op == FLARE_OP_PP_FORWARD ? BH : grp};
    size_t max_acc = 0, max_al = 0;
    for (int gi = 0; gi < 3; ++gi) {
      const EncPlan p = plan_encode(dev, groups[gi], N, M);
      const size_t acc = align256((size_t)groups[gi] * p.pmax * M * D * sizeof(float));
      const size_t al = align256((size_t)groups[gi] * p.pmax * M * sizeof(float2));
      if (acc > max_acc) max_acc = acc;
      if (al > max_al) max_al = al;
    }
    w.part_acc = 0;
    w.part_al = max_acc;
    off = max_acc + max_al;
  }
  if (need_z) { w.z = off; off += align256((size_t)BH * M * D * sizeof(float)); w.l = off; off += align256((size_t)BH * M * sizeof(float)); }
  if (need_q) { w.q = off; off += align256((size_t)BH * M * D * sizeof(float)); }
  w.total = off;
  return w;
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
  if (op < FLARE_OP_ENCODE || op > FLARE_OP_PP_FORWARD) return 0;
  if (op == FLARE_OP_DECODE) return 0;
  Dev dev;
  if (query_dev(dev) != FLARE_OK) return 0;
  const bool need_z = op == FLARE_OP_FORWARD || op == FLARE_OP_PP_FORWARD;
  const bool need_q = op == FLARE_OP_PP_FORWARD;
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
  const EncPlan p = plan_encode(dev, BH, N, M);
  float* pacc = (float*)((char*)ws + w.part_acc);
  float2* pal = (float2*)((char*)ws + w.part_al);
  if (N > 0) {
    rc = launch_encode(dev, Q, dtype, q_batched, K, V, 0, BH, H, N, M, D, dtype, qs, pacc, pal, p, st);
    if (rc) return rc;
  }
  return launch_merge(p, pacc, pal, 0, BH, H, N, M, D, Z, L, nullptr, FLARE_F32, nullptr, nullptr, st);
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
  return launch_decode(dev, Q, dtype, q_batched, K, Z, Y, 0, B * H, H, N, M, D, dtype, qs, (hipStream_t)stream);
}

// Shared by flare_forward and the routing half of flare_pp_forward: encode ->
// merge -> decode per head group.  Q has element type qtype.
static int routing(const Dev& dev, const void* Q, int qtype, int q_batched, const void* K, const void* V, void* Y,
                   float* Z, float* L, int B, int H, int N, int M, int D, int dtype, float qs, char* ws,
                   const WsLayout& w, hipStream_t st) {
  const int BH = B * H;
  const int grp = heads_per_group(BH, N, D, dtype);
  float* pacc = (float*)(ws + w.part_acc);
  float2* pal = (float2*)(ws + w.part_al);
  int rc;
  for (int bh0 = 0; bh0 < BH; bh0 += grp) {
    const int nbh = BH - bh0 < grp ? BH - bh0 : grp;
    const EncPlan p = plan_encode(dev, nbh, N, M);
    if (N > 0) {
      rc = launch_encode(dev, Q, qtype, q_batched, K, V, bh0, nbh, H, N, M, D, dtype, qs, pacc, pal, p, st);
      if (rc) return rc;
    }
    rc = launch_merge(p, pacc, pal, bh0, nbh, H, N, M, D, Z, L, nullptr, FLARE_F32, nullptr, nullptr, st);
    if (rc) return rc;
    rc = launch_decode(dev, Q, qtype, q_batched, K, Z, Y, bh0, nbh, H, N, M, D, dtype, qs, st);
    if (rc) return rc;
  }
  return FLARE_OK;
}

int flare_forward(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z_out, float* L_out,
                  int B, int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                  void* stream) {
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
  if (ws_bytes < w.total || (w.total > 0 && !ws)) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  float* Z = Z_out ? Z_out : (float*)(wsc + w.z);
  float* L = L_out ? L_out : (float*)(wsc + w.l);
  const float qs = pick_scale(scale, D) * kLog2e;
  return routing(dev, Q, dtype, q_batched, K, V, Y, Z, L, B, H, N, M, D, dtype, qs, wsc, w, (hipStream_t)stream);
}

int flare_pp_forward(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                     const void* K, const void* V, void* Y, float* Q_out, float* Z_out, float* L_out, int B, int H,
                     int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, 0);
  if (rc) return rc;
  if (!Qs || !Qf || !gate || (N > 0 && (!Ks || !Vs || !K || !V || !Y))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {Qs, Ks, Vs, Qf, gate, K, V, Y, Q_out, Z_out, L_out, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
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
  // Synthesis encode over all heads, merged straight into the blended queries.
  const EncPlan p = plan_encode(dev, BH, N, M);
  float* pacc = (float*)(wsc + w.part_acc);
  float2* pal = (float2*)(wsc + w.part_al);
  if (N > 0) {
    rc = launch_encode(dev, Qs, dtype, 0, Ks, Vs, 0, BH, H, N, M, D, dtype, qs, pacc, pal, p, st);
    if (rc) return rc;
  }
  rc = launch_merge(p, pacc, pal, 0, BH, H, N, M, D, nullptr, nullptr, Qf, dtype, gate, Qb, st);
  if (rc) return rc;
  // Routing with the per-batch float32 queries.
  return routing(dev, Qb, FLARE_F32, 1, K, V, Y, Z, L, B, H, N, M, D, dtype, qs, wsc, w, st);
}

}  // extern "C"
