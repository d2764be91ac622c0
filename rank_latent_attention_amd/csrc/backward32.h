// backward32.h -- reverse mode of the FLARE encoder / decoder pair for
// float32 inputs and outputs on gfx950.  Included once, by flare.hip, after
// backward.h; it reopens the same unnamed namespace.
//
// The derivative is the one backward.h computes (FLARE++ paper, App. B.5
// "Local backward" with one shard, and the derivative of the decoder's
// softmax over the latents, App. A.1), here in float32 throughout: scores
// u = (s log2 e) q . k in log2 units from float32 operands, every weight
// with its exact shift (2^(u - lse2_n) for the decoder, 2^(u - L_m log2 e)
// for the encoder, so each lies in [0, 1]), and plain float32 sums.  The
// decoder side takes the latents centred over the latents (Zc = Z - mean),
// as backward.h does: dY . Zc_m - delta_n equals dY . Z_m - dY . Y_n exactly,
// without the cancellation of a large common part of the latents.
//
// Launches (one call, one stream; "dec" marks the decoder side, which the
// encoder's backward alone leaves out):
//   center   (dec) Zc = Z - mean over latents (center_kernel of backward.h)
//   stats    (dec) per token: lse2_n = log2 sum_m 2^u_mn and
//                  delta_n = sum_m W_mn dY_n . Zc_m                [B,H,N] f32x2
//   col      (dec) per (head, token split), one lane per latent:
//                  partial dZ_m = sum_n W dY_n, partial dQ_m = sum_n dU k_n
//   sum dZ   dZ = sum of the splits (or the given dZ);
//            cl_m = dZ_m . Z_m - dL_m
//   col      per (head, token split): partial dQ_m += sum_n dS k_n
//   sum dQ   dQ = s sum of the splits (and of the batch for shared queries)
//   row      one lane per token: dK_n = s sum_m (dU + dS) q_m, dV_n = sum_m P dZ_m
// with W = 2^(u - lse2_n), dU = W (dY_n . Zc_m - delta_n),
// P = 2^(u - L_m log2 e), dS = P (dZ_m . V_n - cl_m).
// Every sum runs in a fixed order, so the result is deterministic.

namespace {

constexpr int kTok32 = 1024;    // tokens per workgroup of the statistics and row passes
constexpr int kColTile32 = 64;  // tokens per LDS tile of the col pass

struct B32Args {
  const float* Q;   // [H or B H, M, D] (q_batched)
  const float* K;   // [B,H,N,D]
  const float* V;   // [B,H,N,D] (encoder side)
  const float* Z;   // [B,H,M,D] the forward's latents
  const float* Zc;  // [B,H,M,D] centred latents (decoder side)
  const float* L;   // [B,H,M] the forward's log-normalisers (natural log)
  const float* dY;  // [B,H,N,D] (decoder side)
  const float* dz;  // [B,H,M,D] the latents' cotangent read by the encoder side
  const float* dL;  // [B,H,M] or null
  float2* stats;    // [B,H,N] (lse2_n, delta_n)
  float* part_dz;   // [B H S][M][D]
  float* part_dq;   // [B H S][M][D]
  float* cl;        // [B,H,M]
  float* dz_ws;     // sum dZ: the summed dZ (decoder side), or null
  float* dz_user;   // sum dZ: a copy for the caller, or null
  float* dQ;        // [H or B H, M, D]
  float* dK;        // [B,H,N,D]
  float* dV;        // [B,H,N,D] (not written when alias)
  int q_batched, B, H, N, M, S, accumulate, alias;
  float qscale;  // s log2 e
  float scale;   // s
};

template <int D> __device__ inline void load_row32(float (&x)[D], const float* p) {
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const f32x4 t = reinterpret_cast<const f32x4*>(p)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[4 * i + j] = t[j];
  }
}

// a . b in ascending feature order; b is 16-byte aligned (LDS or global)
template <int D> __device__ inline float dot32(const float (&a)[D], const float* b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const f32x4 t = reinterpret_cast<const f32x4*>(b)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(a[4 * i + j], t[j], s);
  }
  return s;
}

// acc += w * b
template <int D> __device__ inline void axpy32(float (&acc)[D], float w, const float* b) {
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const f32x4 t = reinterpret_cast<const f32x4*>(b)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[4 * i + j] = fmaf(w, t[j], acc[4 * i + j]);
  }
}

template <int D> __device__ inline void store_row32(float* p, const float (&x)[D]) {
#pragma unroll
  for (int i = 0; i < D / 4; ++i)
    reinterpret_cast<f32x4*>(p)[i] = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
}

// Stage rows [M][D] of src into LDS, each value times mul.
__device__ inline void stage32(float* dst, const float* src, int n, float mul) {
  for (int e = threadIdx.x; e < n; e += blockDim.x) dst[e] = src[e] * mul;
}

// ----------------------------------------------------------------------------
// Decoder statistics: one lane per token, the head's scaled queries and
// centred latents in LDS.  Grid (B H, ceil(N / kTok32)).
// ----------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads) stats32_kernel(B32Args a) {
  extern __shared__ __align__(16) float sm32[];
  const int M = a.M, N = a.N;
  float* qs = sm32;
  float* zs = sm32 + (size_t)M * D;
  const int bh = blockIdx.x, h = bh % a.H;
  stage32(qs, a.Q + (size_t)(a.q_batched ? bh : h) * M * D, M * D, a.qscale);
  stage32(zs, a.Zc + (size_t)bh * M * D, M * D, 1.f);
  __syncthreads();
  const int n0 = blockIdx.y * kTok32, n1 = min(N, n0 + kTok32);
  for (int n = n0 + (int)threadIdx.x; n < n1; n += kThreads) {
    const size_t row = ((size_t)bh * N + n) * D;
    float k[D], dy[D];
    load_row32<D>(k, a.K + row);
    load_row32<D>(dy, a.dY + row);
    float mx = -INFINITY;
    for (int m = 0; m < M; ++m) mx = fmaxf(mx, dot32<D>(k, qs + m * D));
    float l = 0.f, t = 0.f;
    for (int m = 0; m < M; ++m) {
      const float w = __builtin_amdgcn_exp2f(dot32<D>(k, qs + m * D) - mx);
      l += w;
      t = fmaf(w, dot32<D>(dy, zs + m * D), t);
    }
    a.stats[(size_t)bh * N + n] = make_float2(mx + __builtin_amdgcn_logf(l), t / l);
  }
}

// ----------------------------------------------------------------------------
// Col pass: one lane per latent (blockDim = M rounded up to 64), token tiles
// of the split in LDS.  Workgroup w = (bh, split) with bh = w / S; split sp
// covers tokens [sp N / S, (sp + 1) N / S).
// ----------------------------------------------------------------------------
template <int D, bool DEC>
__global__ void __launch_bounds__(kThreads) col32_kernel(B32Args a) {
  __shared__ __align__(16) float kt[kColTile32 * D];
  __shared__ __align__(16) float xt[kColTile32 * D];  // dY (decoder side) or V
  __shared__ float2 st[kColTile32];
  const int M = a.M, N = a.N, S = a.S;
  const int bh = blockIdx.x / S, sp = blockIdx.x % S, h = bh % a.H;
  const int n_lo = (int)((long long)sp * N / S), n_hi = (int)((long long)(sp + 1) * N / S);
  const int m = threadIdx.x;
  const bool live = m < M;
  const int mr = live ? m : M - 1;  // lanes past M repeat row M - 1 and store nothing
  float q[D], lat[D], adq[D], adz[D];
  load_row32<D>(q, a.Q + ((size_t)(a.q_batched ? bh : h) * M + mr) * D);
#pragma unroll
  for (int i = 0; i < D; ++i) q[i] *= a.qscale;
  load_row32<D>(lat, (DEC ? a.Zc : a.dz) + ((size_t)bh * M + mr) * D);
  const size_t po = (((size_t)bh * S + sp) * M + mr) * D;
  if (!DEC && a.accumulate) {
    load_row32<D>(adq, a.part_dq + po);
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) adq[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < D; ++i) adz[i] = 0.f;
  const float l2 = DEC ? 0.f : a.L[(size_t)bh * M + mr] * kLog2e;
  const float cl = DEC ? 0.f : a.cl[(size_t)bh * M + mr];
  const float* X = DEC ? a.dY : a.V;
  for (int t0 = n_lo; t0 < n_hi; t0 += kColTile32) {
    const int cnt = min(kColTile32, n_hi - t0);
    __syncthreads();  // the previous tile is consumed
    const size_t base = ((size_t)bh * N + t0) * D / 4;
    for (int e = threadIdx.x; e < cnt * D / 4; e += blockDim.x) {
      reinterpret_cast<f32x4*>(kt)[e] = reinterpret_cast<const f32x4*>(a.K)[base + e];
      reinterpret_cast<f32x4*>(xt)[e] = reinterpret_cast<const f32x4*>(X)[base + e];
    }
    if (DEC)
      for (int e = threadIdx.x; e < cnt; e += blockDim.x) st[e] = a.stats[(size_t)bh * N + t0 + e];
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const float u = dot32<D>(q, kt + j * D);
      if (DEC) {
        const float2 sj = st[j];
        const float w = __builtin_amdgcn_exp2f(u - sj.x);
        const float du = w * (dot32<D>(lat, xt + j * D) - sj.y);
        axpy32<D>(adz, w, xt + j * D);
        axpy32<D>(adq, du, kt + j * D);
      } else {
        const float p = __builtin_amdgcn_exp2f(u - l2);
        const float ds = p * (dot32<D>(lat, xt + j * D) - cl);
        axpy32<D>(adq, ds, kt + j * D);
      }
    }
  }
  if (!live) return;
  store_row32<D>(a.part_dq + po, adq);
  if (DEC) store_row32<D>(a.part_dz + po, adz);
}

// ----------------------------------------------------------------------------
// dZ and cl: one thread per (b, h, m, d); the D threads of a latent are
// consecutive lanes of one wave (D divides 64 and B H M D is a multiple of D).
// With S > 0 splits dZ is their sum (splits in ascending order), else the
// given a.dz.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) sum32_dz_kernel(B32Args a, int D) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)a.B * a.H * a.M * D;
  if (i >= total) return;  // whole latents only (total is a multiple of D)
  const int d = (int)(i % D);
  const size_t r = i / D;  // (bh, m)
  const int M = a.M, S = a.S;
  float dz = 0.f;
  if (a.part_dz) {
    const size_t bh = r / M, m = r % M;
    for (int sp = 0; sp < S; ++sp) dz += a.part_dz[((bh * S + sp) * M + m) * D + d];
  } else {
    dz = a.dz[i];
  }
  if (a.dz_ws) a.dz_ws[i] = dz;
  if (a.dz_user) a.dz_user[i] = dz;
  float c = dz * a.Z[i];
  for (int o = 1; o < D; o <<= 1) c += __shfl_xor(c, o);
  if (d == 0) a.cl[r] = c - (a.dL ? a.dL[r] : 0.f);
}

// dQ = s * sum over the splits (and over the batch for shared queries), one
// thread per (query head, m, d).
__global__ void __launch_bounds__(kThreads) sum32_dq_kernel(B32Args a, int D) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const int QH = a.q_batched ? a.B * a.H : a.H;
  const int M = a.M, S = a.S;
  if (i >= (size_t)QH * M * D) return;
  const int d = (int)(i % D);
  const size_t r = i / D;
  const int m = (int)(r % M), qh = (int)(r / M);
  float s = 0.f;
  const int nb = a.q_batched ? 1 : a.B;
  for (int b = 0; b < nb; ++b) {
    const size_t bh = a.q_batched ? (size_t)qh : (size_t)b * a.H + qh;
    for (int sp = 0; sp < S; ++sp) s += a.part_dq[((bh * S + sp) * M + m) * D + d];
  }
  a.dQ[i] = a.scale * s;
}

// ----------------------------------------------------------------------------
// Row pass: one lane per token; the head's scaled queries, centred latents
// (decoder side), the latents' cotangent, L_m log2 e and cl_m (encoder side)
// in LDS.  Grid (B H, ceil(N / kTok32)).
// ----------------------------------------------------------------------------
template <int D, bool DEC>
__global__ void __launch_bounds__(kThreads) row32_kernel(B32Args a) {
  extern __shared__ __align__(16) float sm32[];
  const int M = a.M, N = a.N;
  const size_t MD = (size_t)M * D;
  float* qs = sm32;
  float* dzs = qs + MD;
  float* zs = dzs + MD;            // decoder side only
  float* l2s = zs + (DEC ? MD : 0);
  float* cls = l2s + M;
  const int bh = blockIdx.x, h = bh % a.H;
  stage32(qs, a.Q + (size_t)(a.q_batched ? bh : h) * MD, (int)MD, a.qscale);
  stage32(dzs, a.dz + (size_t)bh * MD, (int)MD, 1.f);
  if (DEC) stage32(zs, a.Zc + (size_t)bh * MD, (int)MD, 1.f);
  stage32(l2s, a.L + (size_t)bh * M, M, kLog2e);
  stage32(cls, a.cl + (size_t)bh * M, M, 1.f);
  __syncthreads();
  const int n0 = blockIdx.y * kTok32, n1 = min(N, n0 + kTok32);
  for (int n = n0 + (int)threadIdx.x; n < n1; n += kThreads) {
    const size_t row = ((size_t)bh * N + n) * D;
    float k[D], v[D], dy[D], dk[D], dv[D];
    load_row32<D>(k, a.K + row);
    load_row32<D>(v, a.V + row);
    float2 sn = make_float2(0.f, 0.f);
    if (DEC) {
      load_row32<D>(dy, a.dY + row);
      sn = a.stats[(size_t)bh * N + n];
    }
#pragma unroll
    for (int i = 0; i < D; ++i) { dk[i] = 0.f; dv[i] = 0.f; }
    for (int m = 0; m < M; ++m) {
      const float u = dot32<D>(k, qs + m * D);
      float g = 0.f;
      if (DEC) g = __builtin_amdgcn_exp2f(u - sn.x) * (dot32<D>(dy, zs + m * D) - sn.y);
      const float p = __builtin_amdgcn_exp2f(u - l2s[m]);
      g = fmaf(p, dot32<D>(v, dzs + m * D) - cls[m], g);
      axpy32<D>(dv, p, dzs + m * D);
      axpy32<D>(dk, g, qs + m * D);
    }
    // the scaled queries carry s log2 e: dK = s sum g q = ln 2 sum g q_scaled
#pragma unroll
    for (int i = 0; i < D; ++i) dk[i] = dk[i] * kLn2 + (a.alias ? dv[i] : 0.f);
    store_row32<D>(a.dK + row, dk);
    if (!a.alias) store_row32<D>(a.dV + row, dv);
  }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
struct Bwd32Layout {
  size_t zc = 0, stats = 0, part_dz = 0, part_dq = 0, dz = 0, cl = 0, total = 0;
  int S = 0;
};

// Token splits per head of the col passes: about four workgroups per compute
// unit over all heads, at least one tile of tokens per split.
int bwd32_splits(const Dev& dev, int BH, int N) {
  if (N == 0) return 0;
  const long long want = cdiv(4LL * dev.cus, BH), most = cdiv(N, kColTile32);
  return (int)(want < most ? want : most);
}

Bwd32Layout bwd32_layout(const Dev& dev, bool dec, int B, int H, int N, int M, int D) {
  Bwd32Layout w;
  const int BH = B * H;
  w.S = bwd32_splits(dev, BH, N);
  const size_t lat = align256((size_t)BH * M * D * sizeof(float));
  const size_t part = align256((size_t)BH * (w.S > 0 ? w.S : 1) * M * D * sizeof(float));
  size_t off = 0;
  w.part_dq = off; off += part;
  w.cl = off; off += align256((size_t)BH * M * sizeof(float));
  if (dec) {
    w.zc = off; off += lat;
    w.stats = off; off += align256((size_t)BH * (N > 0 ? N : 1) * sizeof(float2));
    w.part_dz = off; off += part;
    w.dz = off; off += lat;
  }
  w.total = off;
  return w;
}

// LDS of the statistics and row passes.
size_t stats32_lds(int D, int M) { return 2 * (size_t)M * D * sizeof(float); }
size_t row32_lds(bool dec, int D, int M) { return ((dec ? 3 : 2) * (size_t)M * D + 2 * (size_t)M) * sizeof(float); }

template <typename K>
int launch_big_lds(K kernel, dim3 grid, size_t lds, hipStream_t st, const B32Args& a) {
  if (lds > 65536 &&
      hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return FLARE_ERR_HIP;
  return launch(kernel, grid, dim3(kThreads), lds, st, a);
}

// The float32 backward.  dec: the FLARE pair (decoder side, then encoder
// side with the dZ it produced); else the encoder alone with the given dZ_in
// (and dL, may be null).  alias: V is K, dK receives dK + dV and dV is not
// written.
int backward32(const Dev& dev, bool dec, const float* Q, int q_batched, const float* K, const float* V,
               const float* Z, const float* L, const float* dY, const float* dZ_in, const float* dL, float* dQ,
               float* dK, float* dV, bool alias, float* dZ_out, int B, int H, int N, int M, int D, float scale,
               char* ws, const Bwd32Layout& w, hipStream_t st) {
  const int BH = B * H;
  B32Args a{};
  a.Q = Q; a.K = K; a.V = V; a.Z = Z; a.L = L; a.dY = dY; a.dL = dL;
  a.part_dq = (float*)(ws + w.part_dq);
  a.cl = (float*)(ws + w.cl);
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.q_batched = q_batched; a.B = B; a.H = H; a.N = N; a.M = M; a.S = w.S;
  a.alias = alias ? 1 : 0;
  a.qscale = scale * kLog2e;
  a.scale = scale;
  const bool d16 = D == 16;
  const unsigned tok_blocks = (unsigned)cdiv(N, kTok32);
  const unsigned col_threads = (unsigned)(64 * cdiv(M, 64));
  int rc;
  if (dec) {
    a.Zc = (float*)(ws + w.zc);
    a.stats = (float2*)(ws + w.stats);
    a.part_dz = (float*)(ws + w.part_dz);
    if (N > 0) {
      rc = launch(center_kernel, dim3(BH), dim3(kThreads), 0, st, Z, (float*)a.Zc, M, D);
      if (rc) return rc;
      rc = launch_big_lds(d16 ? stats32_kernel<16> : stats32_kernel<32>, dim3(BH, tok_blocks), stats32_lds(D, M), st,
                          a);
      if (rc) return rc;
      rc = launch(d16 ? col32_kernel<16, true> : col32_kernel<32, true>, dim3((unsigned)(BH * w.S)),
                  dim3(col_threads), 0, st, a);
      if (rc) return rc;
    }
    a.dz_ws = (float*)(ws + w.dz);
    a.dz_user = dZ_out;
  } else {
    a.part_dz = nullptr;  // dZ is given
    a.dz = dZ_in;
  }
  // dZ (summed, or as given) and cl; with no tokens the decoder's dZ is zero
  rc = launch(sum32_dz_kernel, dim3((unsigned)cdiv((long long)BH * M * D, kThreads)), dim3(kThreads), 0, st, a, D);
  if (rc) return rc;
  if (dec) a.dz = a.dz_ws;
  if (N > 0) {
    a.accumulate = dec ? 1 : 0;
    rc = launch(d16 ? col32_kernel<16, false> : col32_kernel<32, false>, dim3((unsigned)(BH * w.S)),
                dim3(col_threads), 0, st, a);
    if (rc) return rc;
  }
  const int QH = q_batched ? BH : H;
  rc = launch(sum32_dq_kernel, dim3((unsigned)cdiv((long long)QH * M * D, kThreads)), dim3(kThreads), 0, st, a, D);
  if (rc || N == 0) return rc;
  const size_t lds = row32_lds(dec, D, M);
  if (dec) return launch_big_lds(d16 ? row32_kernel<16, true> : row32_kernel<32, true>, dim3(BH, tok_blocks), lds, st, a);
  return launch_big_lds(d16 ? row32_kernel<16, false> : row32_kernel<32, false>, dim3(BH, tok_blocks), lds, st, a);
}

// Workspace of the float32 FLARE++ backward: one region for the synthesis
// recomputation's split partials and the two backward passes (run in that
// order on one stream), then the synthesis latents and log-normalisers, the
// routing queries' cotangent and the synthesis latents' cotangent.
struct PpBwd32Layout {
  size_t region = 0, part_acc = 0, part_al = 0, zs = 0, ls = 0, dq = 0, dqd = 0, total = 0;
};

PpBwd32Layout pp_bwd32_layout(const Dev& dev, int B, int H, int N, int M, int D) {
  PpBwd32Layout w;
  const int BH = B * H;
  const EncPlan p = plan_encode(dev, BH, N, M, FLARE_F32);
  const size_t acc = align256((size_t)BH * p.pmax * M * D * sizeof(float));
  const size_t al = align256((size_t)BH * p.pmax * M * sizeof(float2));
  size_t r = acc + al;
  const size_t r1 = bwd32_layout(dev, true, B, H, N, M, D).total;
  const size_t r2 = bwd32_layout(dev, false, B, H, N, M, D).total;
  r = r > r1 ? r : r1;
  r = r > r2 ? r : r2;
  const size_t lat = align256((size_t)BH * M * D * sizeof(float));
  w.part_acc = 0;
  w.part_al = acc;
  w.zs = r;
  w.ls = w.zs + lat;
  w.dq = w.ls + align256((size_t)BH * M * sizeof(float));
  w.dqd = w.dq + lat;
  w.total = w.dqd + lat;
  return w;
}

bool bwd32_fits(const Dev& dev, bool dec, int D, int M) {
  return row32_lds(dec, D, M) <= dev.lds_max && stats32_lds(D, M) <= dev.lds_max;
}

}  // namespace
