// backward.h -- reverse mode of the FLARE encoder / decoder pair on gfx950
// (bf16 inputs, float32 accumulation).  Included once, by flare.hip, after
// its device helpers and host planning; it reopens the same unnamed
// namespace.
//
// What is computed (FLARE++ paper, App. B.5 "Local backward" with one shard,
// and the derivative of the decoder's softmax over the latents, App. A.1),
// per (b, h), with S = s Q K^T [M x N]:
//   encoder  Z = P V,  P = softmax over tokens,  L = log-normaliser
//            dS_enc = P o (dZ V^T - c + dL),  c_m = dZ_m . Z_m
//            dV = P^T dZ,  dK += s dS_enc^T Q,  dQ += s dS_enc K
//   decoder  Y = W^T Z with W[m,n] = softmax over latents of S[:, n]
//            dS_dec = W o (Z dY^T - delta),  delta_n = dY_n . Y_n
//            dZ = W dY,  dK += s dS_dec^T Q,  dQ += s dS_dec K
// FLARE's backward runs the decoder's part first (it produces dZ) and then
// the encoder's with that dZ (dL = 0).
//
// Scores are in log2 units from the forward's own bf16 operands (Q s log2 e
// rounded, K), so P = 2^(S2 - L log2 e) with the forward's L and
// W = 2^(S2 - lse2_n) with the per-token log2-normaliser of a statistics
// pass: every exponential has its exact shift and lies in [0, 1].
//
// Conditioning.  The latents Z of a long sequence share a large common part
// (each is an average over many tokens), so dY . Z_m - delta_n is a small
// difference of large terms.  The decoder side works on Zc = Z - mean_m Z,
// which changes nothing exactly (the weights of a token sum to one, so
// delta shifts by dY . mean Z as every dY . Z_m does) but makes the bf16
// rounding of the latents relative to their spread.  The encoder side takes
// c_m from the bf16-rounded dZ_m that its score products use, so
// dZ_m . V_n - c_m is the product of that dZ_m with V_n - Z_m.
//
// Launches (one call, one stream):
//   center      Zc = Z - mean over latents                      [B,H,M,D] f32
//   statistics  decode_kernel in statistics mode on Zc: per token
//               -lse2_n and -dY_n . (Y_n - mean Z), as one record of
//               three-part bf16 splits                          [B,H,N] 16 B
//               (the passes add them to score tiles through one extra
//               matrix-core step whose other operand selects the parts)
//   col pass    (decode side) per split of the tokens, lanes = latents:
//               partial sums over tokens of dZ and dQ_dec
//   sum         dZ = sum of splits; c_m from the bf16-rounded dZ_m
//   col pass    (encoder side) partial dQ_enc added onto the decode partials
//   sum         dQ = s * sum of splits (and of the batch for shared queries)
//   row pass    lanes = tokens: dK (both sides) and dV
// The col passes reuse the encode's split plan and LDS tiles (K and the
// second token tensor, DMA-filled, double-buffered, transposing reads for
// the token-contracted products); the row pass reuses the decode's layout
// (the latent-side operands of one head resident in LDS).
namespace {

// ----------------------------------------------------------------------------
// Center the latents of every (b, h): Zc = Z - mean over latents.
// One workgroup per (b, h).
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) center_kernel(const float* Z, float* Zc, int M, int D) {
  __shared__ float red[kThreads];
  __shared__ float mean[32];
  const int t = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * M * D;
  const int RG = kThreads / D;  // row groups
  const int d = t % D;
  float sum = 0.f;
  for (int m = t / D; m < M; m += RG) sum += Z[base + (size_t)m * D + d];
  red[t] = sum;
  __syncthreads();
  if (t < D) {
    float s = 0.f;
    for (int k = 0; k < RG; ++k) s += red[t + k * D];
    mean[t] = s / (float)M;
  }
  __syncthreads();
  for (int e = t; e < M * D; e += kThreads) Zc[base + e] = Z[base + e] - mean[e % D];
}

// ----------------------------------------------------------------------------
// Col pass: lanes own latents (as in the encode), token tiles in LDS.
//   decode side:  per token block, Sw = S2 - lse2 (MFMA accumulator input),
//                 W = 2^Sw, E = Zc dY^T - delta, dS = W o E,
//                 dZ^T += dY^T W^T,  dQ^T += K^T dS^T
//   encoder side: Sp = S2 - L2, P = 2^Sp, E = dZ V^T - c, dS = P o E,
//                 dQ^T += K^T dS^T
// The partial dQ sums are in units of the natural-log scores without the
// factor s (applied by the sum).
// ----------------------------------------------------------------------------
struct ColArgs {
  const void* Q;        // [H,M,D] or [B,H,M,D], type QT (bf16, or float32 routing queries)
  const bf16* K;        // [B,H,N,D]
  const bf16* X;        // decode side: dY; encoder side: V   [B,H,N,D]
  const float* lat;     // decode side: Zc; encoder side: dZ  [B,H,M,D]
  const uint4* srec;    // decode side: per token record (-lse2, -delta)
  const float* L;       // encoder side: the forward's log-normaliser [B,H,M]
  const float* c;       // encoder side: c_m [B,H,M]
  float* part_dz;       // decode side: [BH][pmax][M][D]
  float* part_dq;       // [BH][pmax][M][D]
  long long total;      // BH * N
  int q_batched, H, N, M, nwg, pmax, accumulate;
  float qscale;         // s * log2(e)
};

template <int OFF = 0> __device__ inline bf16x4 tr_read_at(unsigned addr) { return tr_read<OFF>(addr); }

// PV A operand (a transposed token tile, 32 token columns) by transposing reads.
__device__ inline PVOp<bf16> tr_operand(const unsigned (&va)[4], unsigned off, int lane, int D) {
  PVOp<bf16> o;
  const bf16x4 r0 = tr_read_at(va[0] + off), r1 = tr_read_at(va[1] + off);
  const bf16x4 r2 = tr_read_at(va[2] + off), r3 = tr_read_at(va[3] + off);
  o.a0 = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
  o.a1 = __builtin_shufflevector(r2, r3, 0, 1, 2, 3, 4, 5, 6, 7);
  pv_wait(o, lane, D);
  return o;
}

// LDS reads of tiles that a DMA completed before the last barrier, issued
// as inline assembly like the transposing reads: as ordinary loads the
// compiler cannot tell them apart from the DMA into the other buffer (or from
// the statistics prefetch) and makes each wait for all outstanding memory
// operations.  lds_wait() must run before any of them is used.
__device__ inline bf16x8 lds_read16(unsigned addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
template <int D> __device__ inline void lds_wait(QKOp<bf16, D>& a, QKOp<bf16, D>& b, bf16x8& c) {
  if constexpr (D == 32)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a.v[0]), "+v"(a.v[1]), "+v"(b.v[0]), "+v"(b.v[1]), "+v"(c));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a.v[0]), "+v"(b.v[0]), "+v"(c));
}

__device__ inline void pack16(const f32x16& p, bf16x8& b0, bf16x8& b1) {
#pragma unroll
  for (int r = 0; r < 8; ++r) { b0[r] = (bf16)p[r]; b1[r] = (bf16)p[8 + r]; }
}

// B operand of the record step: ones at the three parts of the first (y:
// second) value of a split3_record, in the lanes of k = 0..7; zero elsewhere.
__device__ inline bf16x8 record_select(int g, bool second) {
  bf16x8 r;
  const bf16 one = (bf16)(g == 0 ? 1.f : 0.f), zero = (bf16)0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = ((i & 3) != 3 && (i >= 4) == second) ? one : zero;
  return r;
}

// acc + the record's x (sel = record_select(g, false)) or y on every column:
// the A operand is the row's record, in both halves of the lane's k range.
__device__ inline f32x16 record_add(const uint4& rec, const bf16x8& sel, const f32x16& acc) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(&rec);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sel, acc, 0, 0, 0);
}

__device__ inline float record_value(const uint4& rec, bool second) {
  const bf16x8 r = *reinterpret_cast<const bf16x8*>(&rec);
  const int o = second ? 4 : 0;
  return ((float)r[o] + (float)r[o + 1]) + (float)r[o + 2];
}

__device__ inline f32x16 splat16(float v) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = v;
  return r;
}

template <typename QT, int D, int NW, int WN, bool DEC>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) bwd_col_kernel(ColArgs a) {
  constexpr int ROWS = dma_rows<NW>();
  constexpr int TE = ROWS * D;                       // elements per tile
  constexpr unsigned BUFB = 2 * TE * sizeof(bf16);   // bytes between the two buffers
  constexpr int G = NW / WN;
  static_assert(NW * 64 >= ROWS, "one statistics row per thread");
  __shared__ __align__(16) bf16 tiles[4 * TE];       // [buffer][K, X][TE]
  // decode side: the tile rows' statistics records, [buffer][ROWS]
  __shared__ __align__(16) uint4 srl[DEC ? 2 * ROWS : 1];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int mg = wave % G, ng = wave / G;
  const int N = a.N, M = a.M;
  bf16* const kt0 = tiles;
  bf16* const xt0 = tiles + TE;

  const TileOffs<D> to = tile_offsets<D>(lane);
  const unsigned sra = lds_addr(srl) + (unsigned)li * 16u;  // this lane's record row in buffer 0
  unsigned ka[D / 16], kx[D / 16], va[4], vx[4];
  {
    const unsigned bk = lds_addr(kt0), bx = lds_addr(xt0);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) { ka[s] = bk + to.kq[s]; kx[s] = bx + to.kq[s]; }
#pragma unroll
    for (int k = 0; k < 4; ++k) { va[k] = bk + to.vq[k]; vx[k] = bx + to.vq[k]; }
  }

  long long x = piece_start(blockIdx.x, a.total, a.nwg);
  const long long xe = piece_start(blockIdx.x + 1, a.total, a.nwg);
  while (x < xe) {
    const int bh = (int)(x / N);
    const long long hb = (long long)bh * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int h = bh % a.H;
    const int slot = (blockIdx.x - piece_of(hb, a.total, a.nwg)) * WN + ng;

    // this wave's latent (B operand column): scaled query and latent-side row
    const int m = mg * 32 + li;
    const int mc = m < M ? m : M - 1;
    QKOp<bf16, D> qop, lop;
    load_op_scaled<D>(qop, reinterpret_cast<const QT*>(a.Q) + ((size_t)(a.q_batched ? bh : h) * M + mc) * D, g,
                      a.qscale);
    load_op_scaled<D>(lop, a.lat + ((size_t)bh * M + mc) * D, g, 1.f);
    if (m >= M) { zero_op<D>(qop); zero_op<D>(lop); }
    f32x16 cp = {}, cg = {};
    const bf16x8 sel_s = record_select(g, false), sel_e = record_select(g, true);
    if constexpr (!DEC) {
      // latents past M: shift +inf, so their weights are exactly zero
      cp = splat16(m < M ? -a.L[(size_t)bh * M + m] * kLog2e : -INFINITY);
      cg = splat16(m < M ? -a.c[(size_t)bh * M + m] : 0.f);
    }
    f32x16 accq = {}, accz = {};

    const bf16* Kh = a.K + (size_t)bh * N * D;
    const bf16* Xh = a.X + (size_t)bh * N * D;
    const uint4* Sr = DEC ? a.srec + (size_t)bh * N : nullptr;
    __syncthreads();  // the previous piece is done with the tiles
    dma_tile<D, NW>(kt0, Kh, n_lo, n_hi, wave, lane);
    dma_tile<D, NW>(xt0, Xh, n_lo, n_hi, wave, lane);
    if constexpr (DEC) {
      if ((int)threadIdx.x < ROWS) {
        const int r = n_lo + (int)threadIdx.x;
        srl[threadIdx.x] = Sr[r < n_hi ? r : n_hi - 1];
      }
    }
    wait_dma();
    __syncthreads();
    int buf = 0;
    for (int t0 = n_lo; t0 < n_hi; t0 += ROWS) {
      const int tn = t0 + ROWS;
      uint4 rnext = make_uint4(0, 0, 0, 0);
      if (tn < n_hi) {
        dma_tile<D, NW>(tiles + (buf ^ 1) * 2 * TE, Kh, tn, n_hi, wave, lane);
        dma_tile<D, NW>(tiles + (buf ^ 1) * 2 * TE + TE, Xh, tn, n_hi, wave, lane);
        if constexpr (DEC) {
          if ((int)threadIdx.x < ROWS) {
            const int r = tn + (int)threadIdx.x;
            rnext = Sr[r < n_hi ? r : n_hi - 1];
          }
        }
      }
      for (int nb = ng; nb < ROWS / 32; nb += WN) {
        const int row0 = t0 + 32 * nb;
        if (row0 >= n_hi) break;
        const unsigned off = buf * BUFB + nb * 64 * D;
        QKOp<bf16, D> kop, xop;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          kop.v[s] = lds_read16(ka[s] + off);
          xop.v[s] = lds_read16(kx[s] + off);
        }
        bf16x8 recv = {};
        if constexpr (DEC) recv = lds_read16(sra + (unsigned)(buf * ROWS + 32 * nb) * 16u);
        lds_wait<D>(kop, xop, recv);
        if constexpr (DEC) {
          // the token rows' -lse2 and -delta enter through the record step
          // (A operand row = token li of the block)
          const uint4 rec = *reinterpret_cast<const uint4*>(&recv);
          cp = record_add(rec, sel_s, f32x16{});
          cg = record_add(rec, sel_e, f32x16{});
        }
        f32x16 s = qk_mma<D>(kop, qop, cp);
        const f32x16 e = qk_mma<D>(xop, lop, cg);
        if (row0 + 32 > n_hi) mask_rows(s, n_hi - row0, g);
        f32x16 p, ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(s[r]);
          ds[r] = p[r] * e[r];
        }
        bf16x8 d0, d1;
        pack16(ds, d0, d1);
        accq = pv_mma(tr_operand(va, off, lane, D), d0, d1, accq);
        if constexpr (DEC) {
          bf16x8 w0, w1;
          pack16(p, w0, w1);
          accz = pv_mma(tr_operand(vx, off, lane, D), w0, w1, accz);
        }
      }
      if constexpr (DEC) {
        if (tn < n_hi && (int)threadIdx.x < ROWS) srl[(buf ^ 1) * ROWS + threadIdx.x] = rnext;
      }
      wait_dma();
      __syncthreads();
      buf ^= 1;
    }
    if (m < M) {
      const size_t pi = ((size_t)bh * a.pmax + slot) * M + m;
      float* dq = a.part_dq + pi * D;
      float* dz = DEC ? a.part_dz + pi * D : nullptr;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        if (8 * c4 + 4 * g < D) {
          f32x4 v = {accq[4 * c4], accq[4 * c4 + 1], accq[4 * c4 + 2], accq[4 * c4 + 3]};
          if (a.accumulate) v = v + *reinterpret_cast<const f32x4*>(dq + 8 * c4 + 4 * g);
          *reinterpret_cast<f32x4*>(dq + 8 * c4 + 4 * g) = v;
          if constexpr (DEC) {
            const f32x4 w = {accz[4 * c4], accz[4 * c4 + 1], accz[4 * c4 + 2], accz[4 * c4 + 3]};
            *reinterpret_cast<f32x4*>(dz + 8 * c4 + 4 * g) = w;
          }
        }
      }
    }
    x = hb + n_hi;
  }
}

// ----------------------------------------------------------------------------
// Sums over the splits, in ascending split order.
// ----------------------------------------------------------------------------
struct SumArgs {
  const float* part;    // [BH][pmax][M][D]
  long long total;      // BH * N (piece plan of the col passes)
  int nwg, WN, pmax, B, H, N, M, D;
  // dZ mode: dZ = sum (or dz_in when given), c_m = bf16(dZ_m) . Z_m - dL_m
  const float* dz_in;   // [B,H,M,D] given cotangent of Z, or null
  const float* Z;       // [B,H,M,D]
  const float* dL;      // [B,H,M] or null
  float* dz;            // [B,H,M,D]
  float* c;             // [B,H,M]
  float* dz_out;        // [B,H,M,D] copy for the caller, or null
  // dQ mode: dQ = s * sum (over the batch too when Q is shared)
  float* dq;
  int q_batched;
  float s;
  int* flags;           // [B H] row-pass flags, cleared here (one thread per head)
};

__device__ inline int split_count(const SumArgs& a, int bh) {
  if (a.N == 0) return 0;
  const long long hb = (long long)bh * a.N;
  return (piece_of(hb + a.N - 1, a.total, a.nwg) - piece_of(hb, a.total, a.nwg) + 1) * a.WN;
}

// Splits in ascending order, loaded kSumBatch at a time before any is
// added, so a batch costs one memory round trip.
constexpr int kSumBatch = 8;
__device__ inline float split_sum(const SumArgs& a, int bh, int md) {
  const int cnt = split_count(a, bh);
  if (cnt == 0) return 0.f;
  const float* p = a.part + (size_t)bh * a.pmax * a.M * a.D + md;
  const size_t stride = (size_t)a.M * a.D;
  float s = 0.f;
  for (int i0 = 0; i0 < cnt; i0 += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j) v[j] = p[(size_t)(i0 + j < cnt ? i0 + j : 0) * stride];
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j) asm volatile("" ::"v"(v[j]));
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j) s += i0 + j < cnt ? v[j] : 0.f;
  }
  return s;
}

// One thread per (b, h, m, d); the D threads of a latent are consecutive
// lanes of one wave (D divides 64 and B H M D is a multiple of D).
__global__ void __launch_bounds__(kThreads) sum_dz_kernel(SumArgs a) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long n = (long long)a.B * a.H * a.M * a.D;
  const bool on = i < n;
  const long long ic = on ? i : 0;
  const int bh = (int)(ic / ((long long)a.M * a.D));
  const int md = (int)(ic % ((long long)a.M * a.D));
  const float v = a.dz_in ? a.dz_in[ic] : split_sum(a, bh, md);
  float prod = (float)(bf16)v * a.Z[ic];
  for (int o = 1; o < a.D; o <<= 1) prod += __shfl_xor(prod, o);
  if (on) {
    if (md == 0 && a.flags) a.flags[bh] = 0;
    a.dz[i] = v;
    if (a.dz_out) a.dz_out[i] = v;
    if (md % a.D == 0) {
      const long long row = ic / a.D;
      a.c[row] = prod - (a.dL ? a.dL[row] : 0.f);
    }
  }
}

// One thread per (head of Q, m, d).
__global__ void __launch_bounds__(kThreads) sum_dq_kernel(SumArgs a) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int QH = a.q_batched ? a.B * a.H : a.H;
  if (i >= (long long)QH * a.M * a.D) return;
  const int hq = (int)(i / ((long long)a.M * a.D));
  const int md = (int)(i % ((long long)a.M * a.D));
  float s = 0.f;
  if (a.q_batched) {
    s = split_sum(a, hq, md);
  } else {
    for (int b = 0; b < a.B; ++b) s += split_sum(a, b * a.H + hq, md);
  }
  a.dq[i] = a.s * s;
}

// ----------------------------------------------------------------------------
// Row pass: lanes own tokens (as in the decode); the latent-side operands of
// one head are resident in LDS.  Per latent block of 32:
//   decode side:  W = 2^(S2 - lse2_n), E = Zc dY_n - delta_n, dS = W o E
//   encoder side: P = 2^(S2 - L2_m),   E = dZ V_n - c_m,      dS += P o E,
//                 dV^T += dZ^T P
//   dK^T += (Q s log2 e)^T dS          (dK = that / log2 e)
// ----------------------------------------------------------------------------
struct RowArgs {
  const void* Q;        // type QT
  const bf16* K;
  const bf16* V;        // encoder side
  const bf16* dY;       // decode side
  const float* Zc;      // decode side
  const uint4* srec;    // decode side: per token record (-lse2, -delta)
  const float* dZ;      // encoder side
  const float* L;       // encoder side
  const float* c;       // encoder side
  const float* Zf;      // encoder side: the encoder's latents Z (the factored pass forms c from them)
  const float* dL;      // encoder side: the cotangent of L, or null (the factored pass adds it to c)
  bf16* dK;
  bf16* dV;             // encoder side
  int v_alias;          // encoder side: V is K, so dK receives dK + dV and dV is not written
  int* flags;           // [B H]: heads the factored pass left to the exact-weight pass
  long long total;
  int q_batched, H, N, M, MB, nwg;
  float qscale;
};

template <int D> struct RowLds {
  static constexpr int RST = D + 8;  // row stride (bf16)
  __host__ __device__ static int tst(int MB) { return MB * 32 + 4; }  // transposed stride
  // qs, zr, dzr rows; qt, dzt transposed; per latent record (-L2, -c)
  static size_t bytes(int MB) {
    return (size_t)(3 * MB * 32 * RST + 2 * D * tst(MB)) * sizeof(bf16) + (size_t)MB * 32 * sizeof(uint4);
  }
};

// Row pass with exact per-row shifts: the encoder weights P = 2^(S2 - L2_m)
// from their own exponentials.  It completes only the heads that the
// factored pass (below) flagged, and skips the others.
// NW waves per workgroup share the staged head: at the largest sizes the
// LDS holds one workgroup per compute unit, so 8 waves keep two per SIMD.
template <typename QT, int D, int NW, bool TAIL, bool DEC, bool ENC>
__global__ void __launch_bounds__(NW * 64) bwd_row_kernel(RowArgs a) {
  constexpr int NT = NW * 64;
  using RL = RowLds<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int MB = a.MB, Mp = 32 * MB, M = a.M, N = a.N;
  const int tst = RL::tst(MB);
  bf16* qs = reinterpret_cast<bf16*>(smem);
  bf16* zr = qs + (size_t)Mp * RL::RST;
  bf16* dzr = zr + (size_t)Mp * RL::RST;
  bf16* qt = dzr + (size_t)Mp * RL::RST;
  bf16* dzt = qt + (size_t)D * tst;
  uint4* lrec = reinterpret_cast<uint4*>(dzt + (size_t)D * tst);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  __builtin_assume(MB >= 1);

  long long x = piece_start(blockIdx.x, a.total, a.nwg);
  const long long xe = piece_start(blockIdx.x + 1, a.total, a.nwg);
  while (x < xe) {
    const int bh = (int)(x / N);
    const long long hb = (long long)bh * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int h = bh % a.H;
    if (a.flags[bh] == 0) {  // the factored pass completed this head (uniform over the workgroup)
      x = hb + n_hi;
      continue;
    }

    __syncthreads();  // the previous piece is done with the staged head
    {
      const QT* Qh = reinterpret_cast<const QT*>(a.Q) + (size_t)(a.q_batched ? bh : h) * M * D;
      for (int e = threadIdx.x; e < Mp * D; e += NT) {
        const int m = e / D, d = e % D;
        const bool in = m < M;
        const bf16 q = (bf16)(in ? to_f(Qh[(size_t)m * D + d]) * a.qscale : 0.f);
        qs[m * RL::RST + d] = q;
        qt[d * tst + m] = q;
        if constexpr (DEC) zr[m * RL::RST + d] = (bf16)(in ? a.Zc[((size_t)bh * M + m) * D + d] : 0.f);
        if constexpr (ENC) {
          const bf16 z = (bf16)(in ? a.dZ[((size_t)bh * M + m) * D + d] : 0.f);
          dzr[m * RL::RST + d] = z;
          dzt[d * tst + m] = z;
        }
      }
      if constexpr (ENC) {
        for (int m = threadIdx.x; m < Mp; m += NT) {
          // latents past M: a shift far beyond any score, zero weight
          lrec[m] = m < M ? split3_record(-a.L[(size_t)bh * M + m] * kLog2e, -a.c[(size_t)bh * M + m])
                          : split3_record(-1e30f, 0.f);
        }
      }
    }
    __syncthreads();

    const bf16* Kh = a.K + (size_t)bh * N * D;
    const bf16x8 sel_s = record_select(g, false), sel_e = record_select(g, true);
    for (int t0 = n_lo + 32 * wave; t0 < n_hi; t0 += 32 * NW) {
      // lanes past the piece recompute its last token and store the same values there
      const int n = t0 + li < n_hi ? t0 + li : n_hi - 1;
      QKOp<bf16, D> kop, yop, vop;
      load_op<D>(kop, Kh + (size_t)n * D, g);
      f32x16 cw = {}, cd = {};
      if constexpr (DEC) {
        load_op<D>(yop, a.dY + ((size_t)bh * N + n) * D, g);
        const uint4 rec = a.srec[(size_t)bh * N + n];
        cw = splat16(record_value(rec, false));
        cd = splat16(record_value(rec, true));
      }
      if constexpr (ENC) load_op<D>(vop, a.V + ((size_t)bh * N + n) * D, g);
      f32x16 acck = {}, accv = {};
      for (int mb = 0; mb < MB; ++mb) {
        QKOp<bf16, D> qop;
        load_op<D>(qop, qs + (mb * 32 + li) * RL::RST, g);
        f32x16 ds = {};
        if constexpr (DEC) {
          QKOp<bf16, D> zop;
          load_op<D>(zop, zr + (mb * 32 + li) * RL::RST, g);
          f32x16 s = qk_mma<D>(qop, kop, cw);
          const f32x16 e = qk_mma<D>(zop, yop, cd);
          if (TAIL && mb == MB - 1) mask_rows(s, M - mb * 32, g);
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(s[r]) * e[r];
        }
        if constexpr (ENC) {
          QKOp<bf16, D> zop;
          load_op<D>(zop, dzr + (mb * 32 + li) * RL::RST, g);
          // the latent rows' -L2 and -c through the record step (A operand
          // row = latent li of the block)
          const uint4 rec = lrec[mb * 32 + li];
          const f32x16 s = qk_mma<D>(qop, kop, record_add(rec, sel_s, f32x16{}));
          const f32x16 e = qk_mma<D>(zop, vop, record_add(rec, sel_e, f32x16{}));
          f32x16 p;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(s[r]);
            ds[r] += p[r] * e[r];
          }
          PVOp<bf16> zt;
          if (li < D) load_pv(zt, dzt + li * tst + mb * 32, g);
          else ones_pv(zt, li, D);
          bf16x8 p0, p1;
          pack16(p, p0, p1);
          accv = pv_mma(zt, p0, p1, accv);
        }
        PVOp<bf16> qtop;
        if (li < D) load_pv(qtop, qt + li * tst + mb * 32, g);
        else ones_pv(qtop, li, D);
        bf16x8 d0, d1;
        pack16(ds, d0, d1);
        acck = pv_mma(qtop, d0, d1, acck);
      }
      constexpr float kInvLog2e = 0.69314718055994531f;
      bf16* dk = a.dK + ((size_t)bh * N + n) * D;
      bf16* dv = ENC && !a.v_alias ? a.dV + ((size_t)bh * N + n) * D : nullptr;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        if (8 * c4 + 4 * g < D) {
          bf16x4 u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acck[4 * c4 + i] * kInvLog2e;
            if constexpr (ENC) v += a.v_alias ? accv[4 * c4 + i] : 0.f;
            u[i] = (bf16)v;
          }
          *reinterpret_cast<bf16x4*>(dk + 8 * c4 + 4 * g) = u;
          if (ENC && !a.v_alias) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (bf16)accv[4 * c4 + i];
            *reinterpret_cast<bf16x4*>(dv + 8 * c4 + 4 * g) = v;
          }
        }
      }
    }
    x = hb + n_hi;
  }
}

// ----------------------------------------------------------------------------
// Row pass, factored.  With mu the largest L2_m of the head, the encoder
// weights factor exactly into a per-token, a per-pair and a per-latent part:
//   P[m,n] = 2^(S2 - L2_m) = a_n * W[m,n] * b_m,
//   a_n = 2^(lse2_n - mu),  W = 2^(S2 - lse2_n),  b_m = 2^(mu - L2_m),
// so P needs no exponential or score product of its own.  b_m moves onto
// the staged latent-side rows (dZ' = b_m dZ, c' = b_m c, so
// P o (dZ V^T - c) = a_n W o (dZ' V^T - c')), and a_n is one scalar per
// lane:
//   dS = W o (E_dec + a_n E'),  dV = a_n sum_m W dZ'_m.
// Without the decoder side (the encoder's backward alone) the pass uses
// W = 2^(S2 - mu) and a_n = 1.  The factors stay in range when the head's
// L2 spread is at most kRangeMax and a_n lies in [2^-120, 2^120]; a head
// outside is flagged (flags[bh] = 1) and left to the exact-weight pass.
// ----------------------------------------------------------------------------
constexpr float kRangeMax = 64.f;

template <typename QT, int D, int NW, bool TAIL, bool DEC>
__global__ void __launch_bounds__(NW * 64) bwd_row_fast_kernel(RowArgs a) {
  constexpr int NT = NW * 64;
  using RL = RowLds<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float wred[2][NW];
  __shared__ int next_blk;  // the next unclaimed 32-token block of the piece
  const int MB = a.MB, Mp = 32 * MB, M = a.M, N = a.N;
  const int tst = RL::tst(MB);
  bf16* qs = reinterpret_cast<bf16*>(smem);
  bf16* zr = qs + (size_t)Mp * RL::RST;
  bf16* dzr = zr + (size_t)Mp * RL::RST;
  bf16* qt = dzr + (size_t)Mp * RL::RST;
  bf16* dzt = qt + (size_t)D * tst;
  uint4* crec = reinterpret_cast<uint4*>(dzt + (size_t)D * tst);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  __builtin_assume(MB >= 1);

  long long x = piece_start(blockIdx.x, a.total, a.nwg);
  const long long xe = piece_start(blockIdx.x + 1, a.total, a.nwg);
  while (x < xe) {
    const int bh = (int)(x / N);
    const long long hb = (long long)bh * N;
    const int n_lo = (int)(x - hb);
    const int n_hi = (int)((xe < hb + N ? xe : hb + N) - hb);
    const int h = bh % a.H;
    const float* Lh = a.L + (size_t)bh * M;

    __syncthreads();  // the previous piece is done with the staged head
    // mu and the spread of L2 over the head's latents (every thread ends
    // with the same values: the same reductions in the same order)
    float mx = -INFINITY, mn = INFINITY;
    for (int m = threadIdx.x; m < M; m += NT) {
      const float l2 = Lh[m] * kLog2e;
      mx = fmaxf(mx, l2);
      mn = fminf(mn, l2);
    }
    for (int o = 32; o > 0; o >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o));
      mn = fminf(mn, __shfl_xor(mn, o));
    }
    if (lane == 0) { wred[0][wave] = mx; wred[1][wave] = mn; }
    __syncthreads();
    mx = wred[0][0];
    mn = wred[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) { mx = fmaxf(mx, wred[0][w]); mn = fminf(mn, wred[1][w]); }
    const float mu = mx;
    if (!(mx - mn <= kRangeMax)) {  // also when L holds a non-finite value
      if (threadIdx.x == 0) a.flags[bh] = 1;
      x = hb + n_hi;
      continue;
    }
    {
      const QT* Qh = reinterpret_cast<const QT*>(a.Q) + (size_t)(a.q_batched ? bh : h) * M * D;
      // Mp D is a multiple of NT, so every thread runs every iteration and
      // the D threads of one latent (consecutive lanes) can shuffle
      for (int e = threadIdx.x; e < Mp * D; e += NT) {
        const int m = e / D, d = e % D;
        const bool in = m < M;
        const size_t i = ((size_t)bh * M + (in ? m : 0)) * D + d;
        const bf16 q = (bf16)(in ? to_f(Qh[(size_t)(in ? m : 0) * D + d]) * a.qscale : 0.f);
        qs[m * RL::RST + d] = q;
        qt[d * tst + m] = q;
        if constexpr (DEC) zr[m * RL::RST + d] = (bf16)(in ? a.Zc[i] : 0.f);
        const float b = in ? fast_exp2(mu - Lh[in ? m : 0] * kLog2e) : 0.f;
        const bf16 z = (bf16)(b * a.dZ[i]);
        dzr[m * RL::RST + d] = z;
        dzt[d * tst + m] = z;
        float cp = in ? (float)z * a.Zf[i] : 0.f;
        for (int o = 1; o < D; o <<= 1) cp += __shfl_xor(cp, o);
        if (d == 0) {
          if (a.dL && in) cp -= b * a.dL[(size_t)bh * M + m];  // c' = b (bf16(dZ) . Z - dL)
          crec[m] = split3_record(-cp, 0.f);
        }
      }
    }
    // wave w starts with block w; the waves claim the rest as they finish one,
    // so all of them run to the end of the piece (as in the decode)
    if (threadIdx.x == 0) next_blk = NW;
    __syncthreads();

    const bf16* Kh = a.K + (size_t)bh * N * D;
    const bf16x8 sel = record_select(g, false);
    const int nblk = (n_hi - n_lo + 31) / 32;
    int b = wave;
    while (b < nblk) {
      const int t0 = n_lo + 32 * b;
      int bn = 0;
      if (lane == 0) bn = atomicAdd(&next_blk, 1);
      b = __builtin_amdgcn_readfirstlane(bn);  // the next block, claimed before this one's work
      // lanes past the piece recompute its last token and store the same values there
      const int n = t0 + li < n_hi ? t0 + li : n_hi - 1;
      QKOp<bf16, D> kop, yop, vop;
      load_op<D>(kop, Kh + (size_t)n * D, g);
      load_op<D>(vop, a.V + ((size_t)bh * N + n) * D, g);
      f32x16 cw, cd = {};
      float an = 1.f;
      if constexpr (DEC) {
        load_op<D>(yop, a.dY + ((size_t)bh * N + n) * D, g);
        const uint4 rec = a.srec[(size_t)bh * N + n];
        const float nl = record_value(rec, false);  // -lse2
        cw = splat16(nl);
        cd = splat16(record_value(rec, true));
        an = fast_exp2(-nl - mu);
        if (__builtin_amdgcn_ballot_w64(!(an >= 0x1p-120f && an <= 0x1p120f)) != 0) {
          if (lane == 0) a.flags[bh] = 1;  // the exact-weight pass redoes this head
          continue;
        }
      } else {
        cw = splat16(-mu);
      }
      f32x16 acck = {}, accv = {};
      for (int mb = 0; mb < MB; ++mb) {
        QKOp<bf16, D> qop, zop;
        load_op<D>(qop, qs + (mb * 32 + li) * RL::RST, g);
        load_op<D>(zop, dzr + (mb * 32 + li) * RL::RST, g);
        f32x16 s = qk_mma<D>(qop, kop, cw);
        // E' = dZ' V^T - c' (the latent rows' -c' through the record step)
        f32x16 e = qk_mma<D>(zop, vop, record_add(crec[mb * 32 + li], sel, f32x16{}));
        if constexpr (DEC) {
          QKOp<bf16, D> wop;
          load_op<D>(wop, zr + (mb * 32 + li) * RL::RST, g);
          const f32x16 ed = qk_mma<D>(wop, yop, cd);
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = ed[r] + an * e[r];
        }
        if (TAIL && mb == MB - 1) mask_rows(s, M - mb * 32, g);
        f32x16 w, ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          w[r] = fast_exp2(s[r]);
          ds[r] = w[r] * e[r];
        }
        PVOp<bf16> zt, qtop;
        if (li < D) {
          load_pv(zt, dzt + li * tst + mb * 32, g);
          load_pv(qtop, qt + li * tst + mb * 32, g);
        } else {
          ones_pv(zt, li, D);
          ones_pv(qtop, li, D);
        }
        bf16x8 w0, w1, d0, d1;
        pack16(w, w0, w1);
        pack16(ds, d0, d1);
        accv = pv_mma(zt, w0, w1, accv);
        acck = pv_mma(qtop, d0, d1, acck);
      }
      constexpr float kInvLog2e = 0.69314718055994531f;
      bf16* dk = a.dK + ((size_t)bh * N + n) * D;
      bf16* dv = a.v_alias ? nullptr : a.dV + ((size_t)bh * N + n) * D;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        if (8 * c4 + 4 * g < D) {
          bf16x4 u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acck[4 * c4 + i] * kInvLog2e;
            if (a.v_alias) v += an * accv[4 * c4 + i];
            u[i] = (bf16)v;
          }
          *reinterpret_cast<bf16x4*>(dk + 8 * c4 + 4 * g) = u;
          if (!a.v_alias) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (bf16)(an * accv[4 * c4 + i]);
            *reinterpret_cast<bf16x4*>(dv + 8 * c4 + 4 * g) = v;
          }
        }
      }
    }
    x = hb + n_hi;
  }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
struct BwdLayout {
  size_t zc = 0, srec = 0, part_dz = 0, part_dq = 0, dz = 0, c = 0, flags = 0, total = 0;
};

BwdLayout bwd_layout(const Dev& dev, bool dec, int B, int H, int N, int M, int D) {
  BwdLayout w;
  const int BH = B * H;
  const EncPlan p = plan_encode(dev, BH, N, M, FLARE_BF16);
  const size_t part = align256((size_t)BH * p.pmax * M * D * sizeof(float));
  const size_t lat = align256((size_t)BH * M * D * sizeof(float));
  size_t off = 0;
  w.part_dq = off; off += part;
  w.dz = off; off += lat;
  w.c = off; off += align256((size_t)BH * M * sizeof(float));
  w.flags = off; off += align256((size_t)BH * sizeof(int));
  if (dec) {
    w.zc = off; off += lat;
    w.srec = off; off += align256((size_t)BH * N * sizeof(uint4));
    w.part_dz = off; off += part;
  }
  w.total = off;
  return w;
}

size_t row_lds(int D, int M) {
  const int MB = (int)cdiv(M, 32);
  return D == 16 ? RowLds<16>::bytes(MB) : RowLds<32>::bytes(MB);
}

template <typename QT, int D, int NW, int WN, bool DEC>
int launch_col_k(const ColArgs& a, hipStream_t st) {
  return launch(bwd_col_kernel<QT, D, NW, WN, DEC>, dim3(a.nwg), dim3(NW * 64), 0, st, a);
}

template <typename QT, int D, bool DEC>
int launch_col_d(const ColArgs& a, int NW, int WN, hipStream_t st) {
  if (NW == 8 && WN == 1) return launch_col_k<QT, D, 8, 1, DEC>(a, st);
  if (NW != 4) return FLARE_ERR_UNSUPPORTED;  // no kernel for this split plan
  if (WN == 4) return launch_col_k<QT, D, 4, 4, DEC>(a, st);
  if (WN == 2) return launch_col_k<QT, D, 4, 2, DEC>(a, st);
  return launch_col_k<QT, D, 4, 1, DEC>(a, st);
}

template <typename QT>
int launch_col_q(const ColArgs& a, int D, bool dec, const EncPlan& p, hipStream_t st) {
  if (dec)
    return D == 16 ? launch_col_d<QT, 16, true>(a, p.NW, p.WN, st) : launch_col_d<QT, 32, true>(a, p.NW, p.WN, st);
  return D == 16 ? launch_col_d<QT, 16, false>(a, p.NW, p.WN, st) : launch_col_d<QT, 32, false>(a, p.NW, p.WN, st);
}

// qf32: the queries are float32 (FLARE++ routing), else bf16.
int launch_col(const ColArgs& a, int D, bool dec, bool qf32, const EncPlan& p, hipStream_t st) {
  return qf32 ? launch_col_q<float>(a, D, dec, p, st) : launch_col_q<bf16>(a, D, dec, p, st);
}

constexpr int kRowWaves = 8;

// The factored pass, then the exact-weight pass for the heads it flagged.
template <typename QT, int D, bool TAIL, bool DEC, bool ENC>
int launch_row_k(const RowArgs& a, size_t lds, hipStream_t st) {
  static_assert(ENC, "the row pass always has the encoder side");
  const void* ff = (const void*)bwd_row_fast_kernel<QT, D, kRowWaves, TAIL, DEC>;
  const void* fs = (const void*)bwd_row_kernel<QT, D, kRowWaves, TAIL, DEC, ENC>;
  if (lds > 65536) {
    if (hipFuncSetAttribute(ff, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess ||
        hipFuncSetAttribute(fs, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return FLARE_ERR_HIP;
  }
  const int rc = launch(bwd_row_fast_kernel<QT, D, kRowWaves, TAIL, DEC>, dim3(a.nwg), dim3(kRowWaves * 64), lds, st, a);
  if (rc) return rc;
  return launch(bwd_row_kernel<QT, D, kRowWaves, TAIL, DEC, ENC>, dim3(a.nwg), dim3(kRowWaves * 64), lds, st, a);
}

template <typename QT, int D, bool DEC, bool ENC>
int launch_row_t(const RowArgs& a, size_t lds, hipStream_t st) {
  return (a.M & 31) ? launch_row_k<QT, D, true, DEC, ENC>(a, lds, st)
                    : launch_row_k<QT, D, false, DEC, ENC>(a, lds, st);
}

// Both sides (FLARE, FLARE++ routing; bf16 or float32 queries) or the
// encoder side alone (bf16 queries).
int launch_row(const Dev& dev, RowArgs a, int D, bool dec, bool enc, bool qf32, hipStream_t st) {
  const size_t lds = row_lds(D, a.M);
  if (lds > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  // LDS-resident workgroups per compute unit (160 KB of LDS each)
  const long long per_cu = lds <= 80 * 1024 ? 2 : 1;
  const long long want = (long long)dev.cus * per_cu;
  const long long maxw = cdiv(a.total, 32);
  a.nwg = (int)(want < maxw ? want : maxw);
  if (dec && enc) {
    if (qf32)
      return D == 16 ? launch_row_t<float, 16, true, true>(a, lds, st) : launch_row_t<float, 32, true, true>(a, lds, st);
    return D == 16 ? launch_row_t<bf16, 16, true, true>(a, lds, st) : launch_row_t<bf16, 32, true, true>(a, lds, st);
  }
  if (enc && !qf32)
    return D == 16 ? launch_row_t<bf16, 16, false, true>(a, lds, st) : launch_row_t<bf16, 32, false, true>(a, lds, st);
  return FLARE_ERR_UNSUPPORTED;
}

template <typename QT>
int launch_stats_q(const DecArgs& a, size_t lds, int D, hipStream_t st) {
  const bool tail = a.M & 31;
  if (D == 16)
    return tail ? launch_decode_k<bf16, QT, 16, true, false, true>(a, lds, st)
                : launch_decode_mb<bf16, QT, 16, false, true>(a, lds, st);
  return tail ? launch_decode_k<bf16, QT, 32, true, false, true>(a, lds, st)
              : launch_decode_mb<bf16, QT, 32, false, true>(a, lds, st);
}

int launch_stats(const Dev& dev, const void* Q, bool qf32, int q_batched, const bf16* K, const float* Zc,
                 const bf16* dY, uint4* srec, int BH, int H, int N, int M, int D, float qscale, hipStream_t st) {
  DecArgs a{};
  a.Q = Q; a.K = K; a.Z = Zc; a.Y = nullptr;
  a.total = (long long)BH * N;
  a.q_batched = q_batched; a.H = H; a.N = N; a.M = M; a.MB = (int)cdiv(M, 32); a.bh0 = 0;
  a.qscale = qscale;
  a.qmul = nullptr; a.eps = 0.f;
  a.dY = dY; a.srec = srec;
  const long long want = (long long)dev.cus * kDecWgPerCu;
  const long long maxw = cdiv(a.total, 32);
  a.nwg = (int)(want < maxw ? want : maxw);
  const size_t lds = decode_lds(FLARE_BF16, D, M);
  if (lds > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  return qf32 ? launch_stats_q<float>(a, lds, D, st) : launch_stats_q<bf16>(a, lds, D, st);
}

// The backward of the encoder alone (dec false) or of both sides (FLARE),
// one stream.  Q is float32 when qf32 (FLARE++ routing queries), else bf16.
// dZ_in (encoder alone): the given cotangent of Z; dL: of L.  v_alias
// (encoder alone): V is K, and dK receives the sum of both cotangents.
int backward(const Dev& dev, bool dec, bool enc, const void* Q, bool qf32, int q_batched, const bf16* K,
             const bf16* V, const float* Z, const float* L, const bf16* dY, const float* dZ_in, const float* dL,
             float* dQ, bf16* dK, bf16* dV, bool v_alias, float* dZ_out, int B, int H, int N, int M, int D,
             float scale, char* ws, const BwdLayout& w, hipStream_t st) {
  const int BH = B * H;
  const float qs = scale * kLog2e;
  const EncPlan p = plan_encode(dev, BH, N, M, FLARE_BF16);
  float* part_dq = (float*)(ws + w.part_dq);
  float* dz = (float*)(ws + w.dz);
  float* c = (float*)(ws + w.c);
  int rc;
  SumArgs sa{};
  sa.total = p.total; sa.nwg = p.nwg; sa.WN = p.WN; sa.pmax = p.pmax;
  sa.B = B; sa.H = H; sa.N = N; sa.M = M; sa.D = D;
  sa.Z = Z; sa.dL = dL; sa.dz = dz; sa.c = c; sa.dz_out = dZ_out;
  sa.dq = dQ; sa.q_batched = q_batched; sa.s = scale;
  sa.flags = (int*)(ws + w.flags);
  const unsigned lat_grid = (unsigned)cdiv((long long)BH * M * D, kThreads);
  ColArgs ca{};
  ca.Q = Q; ca.K = K; ca.total = p.total;
  ca.q_batched = q_batched; ca.H = H; ca.N = N; ca.M = M; ca.nwg = p.nwg; ca.pmax = p.pmax;
  ca.qscale = qs; ca.part_dq = part_dq;
  float* zc = dec ? (float*)(ws + w.zc) : nullptr;
  uint4* srec = dec ? (uint4*)(ws + w.srec) : nullptr;
  if (N > 0) {
    if (dec) {
      rc = launch(center_kernel, dim3(BH), dim3(kThreads), 0, st, Z, zc, M, D);
      if (rc) return rc;
      rc = launch_stats(dev, Q, qf32, q_batched, K, zc, dY, srec, BH, H, N, M, D, qs, st);
      if (rc) return rc;
      ColArgs cd = ca;
      cd.X = dY; cd.lat = zc; cd.srec = srec; cd.part_dz = (float*)(ws + w.part_dz);
      cd.accumulate = 0;
      rc = launch_col(cd, D, true, qf32, p, st);
      if (rc) return rc;
      sa.part = cd.part_dz;
    } else {
      sa.dz_in = dZ_in;
    }
  } else {
    sa.dz_in = dZ_in;  // no tokens: no partials (the split sums are empty)
  }
  if (dec || enc) {
    rc = launch(sum_dz_kernel, dim3(lat_grid), dim3(kThreads), 0, st, sa);
    if (rc) return rc;
  }
  if (N > 0 && enc) {
    ColArgs ce = ca;
    ce.X = V; ce.lat = dz; ce.L = L; ce.c = c; ce.accumulate = dec ? 1 : 0;
    rc = launch_col(ce, D, false, qf32, p, st);
    if (rc) return rc;
  }
  SumArgs sq = sa;
  sq.part = part_dq;
  const int QH = q_batched ? BH : H;
  rc = launch(sum_dq_kernel, dim3((unsigned)cdiv((long long)QH * M * D, kThreads)), dim3(kThreads), 0, st, sq);
  if (rc) return rc;
  if (N == 0) return FLARE_OK;
  RowArgs ra{};
  ra.Q = Q; ra.K = K; ra.V = V; ra.dY = dY; ra.Zc = zc; ra.srec = srec; ra.dZ = dz; ra.L = L;
  ra.c = c;
  ra.dK = dK; ra.dV = dV; ra.v_alias = v_alias ? 1 : 0;
  ra.Zf = Z; ra.dL = dL; ra.flags = (int*)(ws + w.flags);
  ra.total = (long long)BH * N;
  ra.q_batched = q_batched; ra.H = H; ra.N = N; ra.M = M; ra.MB = (int)cdiv(M, 32);
  ra.qscale = qs;
  return launch_row(dev, ra, D, dec, enc, qf32, st);
}

// ----------------------------------------------------------------------------
// FLARE++ blend, reverse mode (FLARE++ paper, App. A.4 and B.5): with
// Q[b,h] = Qf[h] + g_h Qd[b,h] and the routing queries' cotangent dQ,
//   dQf[h] = sum_b dQ[b,h],  dg_h = sum_{b,m,d} dQ Qd,  dQd = g_h dQ.
// One workgroup per head; every sum runs in a fixed order.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) blend_backward_kernel(const float* dQ, const float* Qd, const float* gate,
                                                                  float* dQd, float* dQf, float* dgate, int B,
                                                                  int H, int M, int D) {
  __shared__ float red[kThreads];
  const int h = blockIdx.x, t = threadIdx.x;
  const int MD = M * D;
  const float g = gate[h];
  float part = 0.f;
  for (int e = t; e < MD; e += kThreads) {
    float s = 0.f;
    for (int b = 0; b < B; ++b) {
      const size_t i = ((size_t)b * H + h) * MD + e;
      const float dq = dQ[i];
      s += dq;
      part += dq * Qd[i];
      dQd[i] = g * dq;
    }
    dQf[(size_t)h * MD + e] = s;
  }
  red[t] = part;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) dgate[h] = red[0];
}

// Workspace of flare_pp_backward: one region reused by the synthesis
// recomputation, the routing backward and the synthesis backward (they run
// in that order on one stream), then the synthesis latents and
// log-normalisers, the routing queries' cotangent and the synthesis
// latents' cotangent.
struct PpBwdLayout {
  size_t region = 0, zs = 0, ls = 0, dq = 0, dqd = 0, total = 0;
  size_t part_acc = 0, part_al = 0;  // the recomputation's split partials, inside the region
};

PpBwdLayout pp_bwd_layout(const Dev& dev, int B, int H, int N, int M, int D) {
  PpBwdLayout w;
  const int BH = B * H;
  const EncPlan p = plan_encode(dev, BH, N, M, FLARE_BF16);
  const size_t acc = align256((size_t)BH * p.pmax * M * D * sizeof(float));
  const size_t al = align256((size_t)BH * p.pmax * M * sizeof(float2));
  size_t r = acc + al;
  const size_t r1 = bwd_layout(dev, true, B, H, N, M, D).total;
  const size_t r2 = bwd_layout(dev, false, B, H, N, M, D).total;
  r = r > r1 ? r : r1;
  r = r > r2 ? r : r2;
  const size_t lat = align256((size_t)BH * M * D * sizeof(float));
  w.part_acc = 0;
  w.part_al = acc;
  w.region = 0;
  w.zs = r;
  w.ls = w.zs + lat;
  w.dq = w.ls + align256((size_t)BH * M * sizeof(float));
  w.dqd = w.dq + lat;
  w.total = w.dqd + lat;
  return w;
}

// ----------------------------------------------------------------------------
// Backward through the FLARE++ input norms (App. A.3, A.4, Table 2 in A.7).
// With r = (mean_d x^2 + eps)^(-1/2) per row and xh = r x, a norm is
// N(x) = xh * alpha (alpha = 1 for N_0).  Its reverse mode, given the
// cotangent dy of N(x):
//   g = dy * alpha,  dx = r (g - xh mean_d(g xh)),  dalpha = sum_rows dy xh.
// Rows are [bh][R][D]; a row's D / 8 16-byte chunks sit in consecutive lanes.
// ----------------------------------------------------------------------------
constexpr int kNormRows = 4096;  // rows per workgroup of the norm backward (at most)

// y = bf16(N(x)) for nrows rows; the head of row i is (i / R) % H.
template <int D>
__global__ void __launch_bounds__(kThreads) norm_rows_kernel(const bf16* x, bf16* y, const float* alpha,
                                                             long long nrows, int R, int H, float eps) {
  constexpr int CPR = D / 8;
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = t / CPR;
  const int c = (int)(t % CPR);
  const bool live = row < nrows;
  const long long rr = live ? row : 0;  // dead lanes follow row 0 through the shuffles
  const bf16x8 v = reinterpret_cast<const bf16x8*>(x + rr * D)[c];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += (float)v[i] * (float)v[i];
#pragma unroll
  for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o);
  const float r = norm_factor(ss, D, eps);
  const int h = (int)((rr / R) % H);
  float a[8];
  if (alpha) {
    const f32x4* ap = reinterpret_cast<const f32x4*>(alpha + h * D + 8 * c);
    const f32x4 a0 = ap[0], a1 = ap[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = a0[i] * r; a[4 + i] = a1[i] * r; }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = r;
  }
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[i] * a[i]);
  if (live) reinterpret_cast<bf16x8*>(y + rr * D)[c] = o;
}

template <typename G> __device__ inline void load8(const G* p, float (&f)[8]);
template <> __device__ inline void load8(const float* p, float (&f)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
}
template <> __device__ inline void load8(const bf16* p, float (&f)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
}
template <typename G> __device__ inline void store8(G* p, const float (&f)[8]);
template <> __device__ inline void store8(float* p, const float (&f)[8]) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{f[0], f[1], f[2], f[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{f[4], f[5], f[6], f[7]};
}
template <> __device__ inline void store8(bf16* p, const float (&f)[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)f[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}

// In place: g holds the cotangent of N(x) on entry and that of x on exit.
// Workgroup w covers rows [ch kNormRows, +kNormRows) of bh = w / nch (ch =
// w % nch) and writes its partial dalpha to part[w][D] when alpha is given
// (summed in a fixed order, so the result is deterministic).
template <int D, typename G>
__global__ void __launch_bounds__(kThreads) norm_rows_backward_kernel(const bf16* x, G* g, const float* alpha,
                                                                      float* part, int R, int nch, int H,
                                                                      float eps) {
  constexpr int CPR = D / 8, RPP = kThreads / CPR;
  __shared__ float red[kThreads][9];
  const int bh = blockIdx.x / nch, ch = blockIdx.x % nch, h = bh % H;
  const int lr = threadIdx.x / CPR, c = threadIdx.x % CPR;
  const int r0 = ch * kNormRows, r1 = min(R, r0 + kNormRows);
  const int span = (r1 - r0 + RPP - 1) / RPP * RPP;  // whole passes over the live rows
  float a[8], acc[8];
  if (alpha) {
    const f32x4* ap = reinterpret_cast<const f32x4*>(alpha + h * D + 8 * c);
    const f32x4 a0 = ap[0], a1 = ap[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = a0[i]; a[4 + i] = a1[i]; }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 1.f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int r = r0 + lr; r < r0 + span; r += RPP) {  // the same trip count on every lane
    const bool live = r < r1;
    const size_t off = ((size_t)bh * R + (live ? r : r0)) * D + 8 * c;
    float xv[8], gv[8];
    load8(x + off, xv);
    load8(g + off, gv);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += xv[i] * xv[i];
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o);
    const float rn = norm_factor(ss, D, eps);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dot += gv[i] * a[i] * xv[i] * rn;
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) dot += __shfl_xor(dot, o);
    const float mean = dot / (float)D;
    float dx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xh = xv[i] * rn;
      dx[i] = rn * (gv[i] * a[i] - xh * mean);
      if (live) acc[i] += gv[i] * xh;
    }
    if (live) store8(g + off, dx);
  }
  if (!alpha) return;  // uniform over the workgroup
#pragma unroll
  for (int i = 0; i < 8; ++i) red[threadIdx.x][i] = acc[i];
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x, cc = d / 8, i = d % 8;
    float sum = 0.f;
    for (int q = 0; q < RPP; ++q) sum += red[q * CPR + cc][i];
    part[(size_t)blockIdx.x * D + d] = sum;
  }
}

// dalpha[h][d] from the partials of head h's B nch workgroups: one
// workgroup per head; thread (j, d) sums partials j, j + G, ... (G = kThreads
// / D lanes per channel), then the G sums are added in order.
__global__ void __launch_bounds__(kThreads) dalpha_sum_kernel(const float* part, float* dalpha, int B, int H,
                                                              int nch, int D) {
  __shared__ float red[kThreads];
  const int h = blockIdx.x, d = threadIdx.x % D, j = threadIdx.x / D, G = kThreads / D;
  const int np = B * nch;
  float s = 0.f;
  for (int q = j; q < np; q += G) {
    const int b = q / nch, ch = q % nch;
    s += part[((size_t)(b * H + h) * nch + ch) * D + d];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
    for (int q = 0; q < G; ++q) t += red[q * D + threadIdx.x];
    dalpha[(size_t)h * D + threadIdx.x] = t;
  }
}

int launch_norm_rows(const bf16* x, bf16* y, const float* alpha, long long nrows, int R, int H, int D, float eps,
                     hipStream_t st) {
  if (nrows == 0) return FLARE_OK;
  const dim3 grid((unsigned)cdiv(nrows * (D / 8), kThreads));
  if (D == 16) return launch(norm_rows_kernel<16>, grid, dim3(kThreads), 0, st, x, y, alpha, nrows, R, H, eps);
  return launch(norm_rows_kernel<32>, grid, dim3(kThreads), 0, st, x, y, alpha, nrows, R, H, eps);
}

// Rows [BHr][R][D] of cotangent g (float or bf16) with raw inputs x; B is the
// number of row blocks per head (the batch, or 1 for [H, M, D] tensors).
template <typename G>
int launch_norm_rows_backward(const bf16* x, G* g, const float* alpha, float* dalpha, float* part, int B, int H,
                              int R, int D, float eps, hipStream_t st) {
  if (R == 0) {
    if (alpha) {
      return launch(dalpha_sum_kernel, dim3((unsigned)H), dim3(kThreads), 0, st, part, dalpha, B, H, 0, D);
    }
    return FLARE_OK;
  }
  const int nch = (int)cdiv(R, kNormRows);
  const dim3 grid((unsigned)((long long)B * H * nch));
  const int rc = D == 16 ? launch(norm_rows_backward_kernel<16, G>, grid, dim3(kThreads), 0, st, x, g, alpha, part, R,
                                 nch, H, eps)
                         : launch(norm_rows_backward_kernel<32, G>, grid, dim3(kThreads), 0, st, x, g, alpha, part, R,
                                 nch, H, eps);
  if (rc || !alpha) return rc;
  return launch(dalpha_sum_kernel, dim3((unsigned)H), dim3(kThreads), 0, st, part, dalpha, B, H, nch, D);
}

struct PpBwdNormLayout {
  size_t pp = 0, qs = 0, ks = 0, k = 0, part = 0, total = 0;
};

// The FLARE++ backward's workspace, then the normalised seeds and keys (bf16)
// and the per-workgroup dalpha partials.
PpBwdNormLayout pp_bwd_norm_layout(const Dev& dev, int B, int H, int N, int M, int D) {
  PpBwdNormLayout w;
  w.pp = 0;
  w.qs = align256(pp_bwd_layout(dev, B, H, N, M, D).total);
  w.ks = w.qs + align256((size_t)H * M * D * sizeof(bf16));
  const size_t tok = align256((size_t)B * H * N * D * sizeof(bf16));
  w.k = w.ks + tok;
  w.part = w.k + tok;
  const long long nch = cdiv(N > M ? N : M, kNormRows);
  w.total = w.part + align256((size_t)B * H * (nch > 0 ? nch : 1) * D * sizeof(float));
  return w;
}

}  // namespace

#include "backward32.h"

// ----------------------------------------------------------------------------
// C ABI of the backward
// ----------------------------------------------------------------------------
extern "C" {

int flare_backward(const void* Q, int q_batched, const void* K, const void* V, const float* Z, const float* L,
                   const void* dY, float* dQ, void* dK, void* dV, float* dZ_out, int B, int H, int N, int M, int D,
                   int dtype, float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, q_batched);
  if (rc) return rc;
  if (!Q || !Z || !L || !dQ || (N > 0 && (!K || !V || !dY || !dK || !dV))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {Q, K, V, Z, L, dY, dQ, dK, dV, dZ_out, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (dtype == FLARE_F32) {
    if (!bwd32_fits(dev, true, D, M)) return FLARE_ERR_UNSUPPORTED;
    const Bwd32Layout w = bwd32_layout(dev, true, B, H, N, M, D);
    if (ws_bytes < w.total || !ws) return FLARE_ERR_WORKSPACE;
    return backward32(dev, true, (const float*)Q, q_batched, (const float*)K, (const float*)V, Z, L,
                      (const float*)dY, nullptr, nullptr, dQ, (float*)dK, (float*)dV, false, dZ_out, B, H, N, M, D,
                      pick_scale(scale, D), (char*)ws, w, (hipStream_t)stream);
  }
  if (row_lds(D, M) > dev.lds_max || decode_lds(FLARE_BF16, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const BwdLayout w = bwd_layout(dev, true, B, H, N, M, D);
  if (ws_bytes < w.total || !ws) return FLARE_ERR_WORKSPACE;
  return backward(dev, true, true, Q, false, q_batched, (const bf16*)K, (const bf16*)V, Z, L, (const bf16*)dY,
                  nullptr, nullptr, dQ, (bf16*)dK, (bf16*)dV, false, dZ_out, B, H, N, M, D, pick_scale(scale, D),
                  (char*)ws, w, (hipStream_t)stream);
}

int flare_encode_backward(const void* Q, int q_batched, const void* K, const void* V, const float* Z, const float* L,
                          const float* dZ, const float* dL, float* dQ, void* dK, void* dV, int B, int H, int N, int M,
                          int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, q_batched);
  if (rc) return rc;
  if (!Q || !Z || !L || !dZ || !dQ || (N > 0 && (!K || !V || !dK || !dV))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {Q, K, V, Z, L, dZ, dL, dQ, dK, dV, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (dtype == FLARE_F32) {
    if (!bwd32_fits(dev, false, D, M)) return FLARE_ERR_UNSUPPORTED;
    const Bwd32Layout w = bwd32_layout(dev, false, B, H, N, M, D);
    if (ws_bytes < w.total || !ws) return FLARE_ERR_WORKSPACE;
    return backward32(dev, false, (const float*)Q, q_batched, (const float*)K, (const float*)V, Z, L, nullptr, dZ, dL,
                      dQ, (float*)dK, (float*)dV, false, nullptr, B, H, N, M, D, pick_scale(scale, D), (char*)ws, w,
                      (hipStream_t)stream);
  }
  if (row_lds(D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const BwdLayout w = bwd_layout(dev, false, B, H, N, M, D);
  if (ws_bytes < w.total || !ws) return FLARE_ERR_WORKSPACE;
  return backward(dev, false, true, Q, false, q_batched, (const bf16*)K, (const bf16*)V, Z, L, nullptr, dZ, dL, dQ,
                  (bf16*)dK, (bf16*)dV, false, nullptr, B, H, N, M, D, pick_scale(scale, D), (char*)ws, w,
                  (hipStream_t)stream);
}

int flare_pp_backward(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                      const void* K, const void* V, const float* Q, const float* Z, const float* L, const void* dY,
                      float* dQs, void* dKs, void* dVs, float* dQf, float* dgate, float* dQ_out, void* dK, void* dV,
                      int B, int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_common(B, H, N, M, D, dtype, 0);
  if (rc) return rc;
  const bool alias = Ks == Vs;
  if (!Qs || !Qf || !gate || !Q || !Z || !L || !dQs || !dQf || !dgate) return FLARE_ERR_INVALID_ARG;
  if (N > 0 && (!Ks || !Vs || !K || !V || !dY || !dKs || (!alias && !dVs) || !dK || !dV)) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {Qs, Ks, Vs, Qf, gate, K, V, Q, Z, L, dY, dQs, dKs, dVs, dQf, dgate, dQ_out, dK, dV, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  if (dtype == FLARE_F32) {
    if (!bwd32_fits(dev, true, D, M)) return FLARE_ERR_UNSUPPORTED;
    const PpBwd32Layout w = pp_bwd32_layout(dev, B, H, N, M, D);
    if (ws_bytes < w.total || !ws) return FLARE_ERR_WORKSPACE;
    char* wsc = (char*)ws;
    hipStream_t st = (hipStream_t)stream;
    const float s = pick_scale(scale, D);
    const int BH = B * H;
    float* Zs = (float*)(wsc + w.zs);
    float* Ls = (float*)(wsc + w.ls);
    float* dQb = dQ_out ? dQ_out : (float*)(wsc + w.dq);
    float* dQd = (float*)(wsc + w.dqd);
    // 1. the synthesis latents Qd = SDPA(Qs, Ks, Vs) and their log-normalisers
    const EncPlan p = plan_encode(dev, BH, N, M, FLARE_F32);
    if (N > 0) {
      rc = launch_encode(Qs, FLARE_F32, 0, Ks, Vs, 0, H, N, M, D, FLARE_F32, s * kLog2e, (float*)(wsc + w.part_acc),
                         (float2*)(wsc + w.part_al), p, Norms{}, st);
      if (rc) return rc;
    }
    rc = launch_merge(p, (float*)(wsc + w.part_acc), (float2*)(wsc + w.part_al), 0, BH, H, N, M, D, Zs, Ls, nullptr,
                      FLARE_F32, nullptr, nullptr, 0, nullptr, 0.f, st);
    if (rc) return rc;
    // 2. the routing pair's backward with the per-batch queries
    rc = backward32(dev, true, Q, 1, (const float*)K, (const float*)V, Z, L, (const float*)dY, nullptr, nullptr, dQb,
                    (float*)dK, (float*)dV, false, nullptr, B, H, N, M, D, s, wsc + w.region,
                    bwd32_layout(dev, true, B, H, N, M, D), st);
    if (rc) return rc;
    // 3. the blend
    rc = launch(blend_backward_kernel, dim3(H), dim3(kThreads), 0, st, dQb, Zs, gate, dQd, dQf, dgate, B, H, M, D);
    if (rc) return rc;
    // 4. the synthesis encoder's backward with dZ = dQd (dL = 0), the seeds
    //    shared over the batch
    return backward32(dev, false, (const float*)Qs, 0, (const float*)Ks, (const float*)Vs, Zs, Ls, nullptr, dQd,
                      nullptr, dQs, (float*)dKs, (float*)dVs, alias, nullptr, B, H, N, M, D, s, wsc + w.region,
                      bwd32_layout(dev, false, B, H, N, M, D), st);
  }
  if (dtype != FLARE_BF16) return FLARE_ERR_UNSUPPORTED;
  if (row_lds(D, M) > dev.lds_max || decode_lds(FLARE_BF16, D, M) > dev.lds_max) return FLARE_ERR_UNSUPPORTED;
  const PpBwdLayout w = pp_bwd_layout(dev, B, H, N, M, D);
  if (ws_bytes < w.total || !ws) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const float s = pick_scale(scale, D);
  const int BH = B * H;
  float* Zs = (float*)(wsc + w.zs);
  float* Ls = (float*)(wsc + w.ls);
  float* dQb = dQ_out ? dQ_out : (float*)(wsc + w.dq);
  float* dQd = (float*)(wsc + w.dqd);
  // 1. the synthesis latents Qd = SDPA(Qs, Ks, Vs) and their log-normalisers
  const EncPlan p = plan_encode(dev, BH, N, M, FLARE_BF16);
  if (N > 0) {
    rc = launch_encode(Qs, FLARE_BF16, 0, Ks, Vs, 0, H, N, M, D, FLARE_BF16, s * kLog2e, (float*)(wsc + w.part_acc),
                       (float2*)(wsc + w.part_al), p, Norms{}, st);
    if (rc) return rc;
  }
  rc = launch_merge(p, (float*)(wsc + w.part_acc), (float2*)(wsc + w.part_al), 0, BH, H, N, M, D, Zs, Ls, nullptr,
                    FLARE_F32, nullptr, nullptr, 0, nullptr, 0.f, st);
  if (rc) return rc;
  // 2. the routing pair's backward with the float32 per-batch queries
  const BwdLayout wr = bwd_layout(dev, true, B, H, N, M, D);
  rc = backward(dev, true, true, Q, true, 1, (const bf16*)K, (const bf16*)V, Z, L, (const bf16*)dY, nullptr, nullptr,
                dQb, (bf16*)dK, (bf16*)dV, false, nullptr, B, H, N, M, D, s, wsc + w.region, wr, st);
  if (rc) return rc;
  // 3. the blend
  rc = launch(blend_backward_kernel, dim3(H), dim3(kThreads), 0, st, dQb, Zs, gate, dQd, dQf, dgate, B, H, M, D);
  if (rc) return rc;
  // 4. the synthesis encoder's backward with dZ = dQd (dL = 0), the seeds
  //    shared over the batch
  const BwdLayout we = bwd_layout(dev, false, B, H, N, M, D);
  return backward(dev, false, true, Qs, false, 0, (const bf16*)Ks, (const bf16*)Vs, Zs, Ls, nullptr, dQd, nullptr,
                  dQs, (bf16*)dKs, (bf16*)dVs, alias, nullptr, B, H, N, M, D, s, wsc + w.region, we, st);
}

int flare_pp_backward_norm(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                           const void* K, const void* V, const float* Q, const float* Z, const float* L,
                           const void* dY, float* dQs, void* dKs, void* dVs, float* dQf, float* dgate, float* dQ_out,
                           void* dK, void* dV, float* dalpha_qs, float* dalpha_ks, float* dalpha_k, int B, int H,
                           int N, int M, int D, int dtype, float scale, int norm_flags, const float* alpha_qs,
                           const float* alpha_ks, const float* alpha_k, float eps, void* ws, size_t ws_bytes,
                           void* stream) {
  if (norm_flags & ~FLARE_NORM_ALL) return FLARE_ERR_INVALID_ARG;
  if (norm_flags == 0)
    return flare_pp_backward(Qs, Ks, Vs, Qf, gate, K, V, Q, Z, L, dY, dQs, dKs, dVs, dQf, dgate, dQ_out, dK, dV, B, H,
                             N, M, D, dtype, scale, ws, ws_bytes, stream);
  int rc = check_common(B, H, N, M, D, dtype, 0);
  if (rc) return rc;
  if (dtype != FLARE_BF16) return FLARE_ERR_UNSUPPORTED;
  if (!(eps > 0.f)) return FLARE_ERR_INVALID_ARG;
  const bool nqs = norm_flags & FLARE_NORM_QS, nks = norm_flags & FLARE_NORM_KS;
  const bool nqf = norm_flags & FLARE_NORM_QF, nk = norm_flags & FLARE_NORM_K;
  const float* aqs = nqs ? alpha_qs : nullptr;
  const float* aks = nks ? alpha_ks : nullptr;
  const float* ak = nk ? alpha_k : nullptr;
  if ((aqs && !dalpha_qs) || (aks && !dalpha_ks) || (ak && !dalpha_k)) return FLARE_ERR_INVALID_ARG;
  if (!Qs || !Qf || (N > 0 && (!Ks || !K))) return FLARE_ERR_INVALID_ARG;
  const void* ptrs[] = {aqs, aks, ak, aqs ? dalpha_qs : nullptr, aks ? dalpha_ks : nullptr, ak ? dalpha_k : nullptr};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FLARE_ERR_INVALID_ARG;
  Dev dev;
  if ((rc = query_dev(dev))) return rc;
  const PpBwdNormLayout w = pp_bwd_norm_layout(dev, B, H, N, M, D);
  if (ws_bytes < w.total || !ws || !aligned16(ws)) return FLARE_ERR_WORKSPACE;
  char* wsc = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const bool alias = Ks == Vs;
  // 1. the normalised inputs the forward used (bf16, like the inputs); Qf is
  //    not needed: the FLARE++ backward takes the routing queries Q as given
  const void* Qs_n = Qs;
  const void* Ks_n = Ks;
  const void* K_n = K;
  if (nqs) {
    rc = launch_norm_rows((const bf16*)Qs, (bf16*)(wsc + w.qs), aqs, (long long)H * M, M, H, D, eps, st);
    if (rc) return rc;
    Qs_n = wsc + w.qs;
  }
  if (nks) {
    rc = launch_norm_rows((const bf16*)Ks, (bf16*)(wsc + w.ks), aks, (long long)B * H * N, N, H, D, eps, st);
    if (rc) return rc;
    Ks_n = wsc + w.ks;
  }
  if (nk) {
    rc = launch_norm_rows((const bf16*)K, (bf16*)(wsc + w.k), ak, (long long)B * H * N, N, H, D, eps, st);
    if (rc) return rc;
    K_n = wsc + w.k;
  }
  // 2. the FLARE++ backward on them; shared synthesis values are the
  //    normalised keys, so their cotangent joins the keys' before step 3
  rc = flare_pp_backward(Qs_n, Ks_n, alias ? Ks_n : Vs, Qf, gate, K_n, V, Q, Z, L, dY, dQs, dKs, dVs, dQf, dgate,
                         dQ_out, dK, dV, B, H, N, M, D, dtype, scale, ws, w.qs, stream);
  if (rc) return rc;
  // 3. each norm's backward, in place on the cotangents
  float* part = (float*)(wsc + w.part);
  if (nqs && (rc = launch_norm_rows_backward((const bf16*)Qs, dQs, aqs, dalpha_qs, part, 1, H, M, D, eps, st)))
    return rc;
  if (nqf && (rc = launch_norm_rows_backward((const bf16*)Qf, dQf, (const float*)nullptr, nullptr, part, 1, H, M, D,
                                              eps, st)))
    return rc;
  if (nks && (rc = launch_norm_rows_backward((const bf16*)Ks, (bf16*)dKs, aks, dalpha_ks, part, B, H, N, D, eps, st)))
    return rc;
  if (nk && (rc = launch_norm_rows_backward((const bf16*)K, (bf16*)dK, ak, dalpha_k, part, B, H, N, D, eps, st)))
    return rc;
  return FLARE_OK;
}

}  // extern "C"
