// proj.h -- the FLARE / FLARE++ encode fed by the block input X: the per-head
// input projections K_h = X W_K,h and V_h = X W_V,h (FLARE++ paper, Sec. 3.1
// "FLARE: fixed-query latent routing") are formed in the encode's tile
// prologue on the matrix cores, from X tiles that arrive by LDS DMA.  The
// projected values never leave LDS; the projected keys are written once, for
// the decode.  Included once, by flare.hip, after backward.h; it reopens the
// same unnamed namespace.
//
// Per 128-token tile of a workgroup's piece (one head):
//   1. the X tile [128][C] is in LDS (its DMA was issued during the previous
//      tile's attention); W_K,h^T and W_V,h^T [D][C] were staged once per head;
//   2. every wave forms 32x32 blocks of K^T = W_K^T X^T and V^T = W_V^T X^T
//      (C / 16 products each) and stores them as bf16 rows into the key and
//      value tiles, in the layout the attention loop reads;
//   3. (with NK) the key rows are N_0-normalised in place; the tile's largest
//      key norm is taken and its keys are written to the key output;
//   4. the next X tile's DMA is issued and the attention loop of the plain
//      bf16 encode (encode_tile) consumes the key and value tiles.
// A workgroup whose exactness check fails (see kScoreErr2) projects its
// tiles again and the waves concerned redo their scores exactly from them.
namespace {

constexpr int kProjC = 128;           // channels of the block input
constexpr int kProjCPR = kProjC / 8;  // 16-byte chunks per input row

struct ProjArgs {
  EncArgs e;       // queries, split partials, plan and norms (e.K, e.V unused)
  const bf16* X;   // [B, N, C], shared by the heads
  const bf16* WK;  // [H, C, D]
  const bf16* WV;  // [H, C, D]; equal to WK when the values are the keys (App. A.6)
  bf16* Kout;      // [B, H, N, D] or null: the projected keys (N_0-normalised with NK)
};

// Swizzled [rows][C] tile of the block input: chunk c of row n sits at chunk
// n C/8 + (c ^ (n & 15)), so the 16 rows of one read pass hit distinct banks.
__device__ inline int xchunk(int n, int c) { return n * kProjCPR + (c ^ (n & (kProjCPR - 1))); }

// DMA of rows [t0, t0 + dma_rows<NW>()) of X_b into the swizzled tile; rows
// at or beyond n_hi repeat row n_hi - 1 (masked out by the attention loop).
template <int NW>
__device__ inline void dma_x(bf16* xt, const bf16* Xb, int t0, int n_hi, int wave, int lane) {
  constexpr int INSTR = dma_rows<NW>() * kProjCPR / 64;  // 64 chunks (1 KB) per wave instruction
  for (int i = wave; i < INSTR; i += NW) {
    const int P = i * 64 + lane;
    const int n = P / kProjCPR;
    const int c = (P % kProjCPR) ^ (n & (kProjCPR - 1));
    int row = t0 + n;
    row = row < n_hi ? row : n_hi - 1;
    __builtin_amdgcn_global_load_lds((const void*)(Xb + (size_t)row * kProjC + c * 8), (lds_void*)(xt + i * 512),
                                     16, 0, 0);
  }
}

// W_0^T (and W_1^T when nm == 2) of one head into LDS as [nm][D][C] with the
// chunk swizzle of xchunk on the D rows.  W is [C][D] in memory.
template <int D, int NW>
__device__ inline void stage_wt(bf16* wt, const bf16* W0, const bf16* W1, int nm) {
  const int chunks = nm * D * kProjCPR;
  for (int q = threadIdx.x; q < chunks; q += NW * 64) {
    const int m = q / (D * kProjCPR), d = (q / kProjCPR) % D, c = q % kProjCPR;
    const bf16* W = m ? W1 : W0;
    bf16x8 v;
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = W[(size_t)(8 * c + s) * D + d];
    reinterpret_cast<bf16x8*>(wt)[(m * D + d) * kProjCPR + (c ^ (d & (kProjCPR - 1)))] = v;
  }
}

// Step 2: 32x32 blocks of K^T (and V^T) of the tile, block t = (matrix t % nm,
// token block t / nm), spread over the waves.  A operand: W^T rows (lane =
// output feature); B operand: X^T columns (lane = token); the accumulator
// lane holds 16 features of its token, stored as four runs of four.
// kerr2 keeps the largest squared norm of a projected key row's rounding
// error, |bf16(k) - k|^2; with klo given, the rounding of that remainder is
// stored there (the keys' low parts, same layout as kt).
template <int D, int NW>
__device__ inline void project_tile(const bf16* xt, const bf16* wt, bf16* kt, bf16* vt, int nm, int wave, int lane,
                                    float& kerr2, bf16* klo = nullptr) {
  static_assert(D == 32, "the projection forms 32 output features per block");
  constexpr int NB = dma_rows<NW>() / 32;
  // operand offsets from an index opaque to the compiler: recomputed here
  // rather than hoisted out of the tile loop, where they would be spilled
  int lid = lane;
  asm volatile("" : "+v"(lid));
  const int li = lid & 31, g = lid >> 5;
  for (int t = wave; t < nm * NB; t += NW) {
    const int m = t % nm, r = 32 * (t / nm) + li;
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < kProjC / 16; ++st) {
      const int c = 2 * st + g;
      const bf16x8 wa = reinterpret_cast<const bf16x8*>(wt)[(m * D + li) * kProjCPR + (c ^ (li & (kProjCPR - 1)))];
      const bf16x8 xb = reinterpret_cast<const bf16x8*>(xt)[xchunk(r, c)];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xb, acc, 0, 0, 0);
    }
    bf16* dst = m ? vt : kt;
    float e2 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 v, vl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = (bf16)acc[4 * j + i];
        const float rem = acc[4 * j + i] - (float)v[i];
        vl[i] = (bf16)rem;
        e2 += rem * rem;
      }
      *reinterpret_cast<bf16x4*>(dst + tile_off<D>(r, 8 * j + 4 * g)) = v;
      if (klo && m == 0) *reinterpret_cast<bf16x4*>(klo + tile_off<D>(r, 8 * j + 4 * g)) = vl;
    }
    if (m == 0) kerr2 = fmaxf(kerr2, pair_sum(e2));  // the other half of the token's row is in lane +-32
  }
}

// The exact recomputation of one wave's share of a tile held in LDS (keys and
// values already projected): token blocks ng, ng + WN, ... with exact scores
// and the online maximum, as encode_careful does from global memory.
// With klo given (keys projected in this call, not normalised), the scores
// also take the keys' low parts: q_hi k_hi + q_lo k_hi + q_hi k_lo.
template <int D>
__device__ inline void careful_tile_lds(const bf16* kt, const bf16* klo, const bf16* vt, int t0, int n_hi, int ng,
                                        int WN, int rows, int lane, const QKOp<bf16, D>& qhi,
                                        const QKOp<bf16, D>& qlo, f32x16& negs, bool& started, float& lsum,
                                        f32x16& acc) {
  const int li = lane & 31, g = lane >> 5;
  for (int nb = ng; nb < rows / 32; nb += WN) {
    const int row0 = t0 + 32 * nb;
    if (row0 >= n_hi) break;
    QKOp<bf16, D> kop;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      kop.v[st] = reinterpret_cast<const bf16x8*>(kt)[chunk_pos<D>(32 * nb + li, 2 * st + g)];
    PVOp<bf16> vop;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int n = 32 * nb + acc_row(j, g);
      const bf16 v = (li < D && row0 + acc_row(j, g) < n_hi) ? vt[tile_off<D>(n, li)] : (bf16)0.f;
      if (j < 8) vop.a0[j] = v;
      else vop.a1[j - 8] = v;
    }
    f32x16 sc = qk_mma<D>(kop, qlo, qk_mma<D>(kop, qhi, negs));
    if (klo) {
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        kop.v[st] = reinterpret_cast<const bf16x8*>(klo)[chunk_pos<D>(32 * nb + li, 2 * st + g)];
      sc = qk_mma<D>(kop, qhi, sc);
    }
    if (row0 + 32 > n_hi) mask_rows(sc, n_hi - row0, g);
    online_step(sc, negs, started, lsum, acc);
    bf16x8 b0, b1;
    lsum += pack_exps(sc, b0, b1);
    acc = pv_mma(vop, b0, b1, acc);
  }
}

// bf16 encode from the block input: NW waves in WN token lanes of G = NW / WN
// latent groups, as encode_dma_kernel; one X tile, one key tile and one value
// tile in LDS (the projection of tile t + 1 waits for the attention of tile
// t, its X DMA does not).  64 KB of LDS per workgroup: two workgroups per
// compute unit, so 8-wave workgroups keep four waves per SIMD and 4-wave
// ones two.
template <typename QT, int D, int NW, int WN, bool NK>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 2, 8)))
encode_proj_kernel(ProjArgs pa) {
  constexpr int ROWS = dma_rows<NW>();
  constexpr int TE = ROWS * D;
  constexpr int G = NW / WN;
  __shared__ __align__(16) bf16 xt[ROWS * kProjC];   // block input tile
  __shared__ __align__(16) bf16 wt[2 * D * kProjC];  // W_K^T, W_V^T of the head
  __shared__ __align__(16) bf16 kv[2 * TE];          // projected key and value tiles
  __shared__ __align__(16) bf16 kl[TE];              // the keys' low parts (exact recomputation only)
  __shared__ float kred[NW], ered[NW];
  __shared__ int cred[NW];
  bf16* const kt = kv;
  bf16* const vt = kv + TE;
  const EncArgs& a = pa.e;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31, g = lane >> 5;
  const int mg = wave % G, ng = wave / G;
  const int N = a.N, M = a.M;
  const bool alias = pa.WV == pa.WK;
  const int nm = alias ? 1 : 2;

  const TileOffs<D> to = tile_offsets<D>(lane);
  const unsigned wofs = ng * 64 * D;
  unsigned ka[D / 16], va[4];
  {
    const unsigned bk = lds_addr(kt) + wofs, bv = lds_addr(alias ? kt : vt) + wofs;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) ka[st] = bk + to.kq[st];
#pragma unroll
    for (int k = 0; k < 4; ++k) va[k] = bv + to.vq[k];
  }

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

    auto qrow = [&]() {
      const int m = mg * 32 + li;
      return reinterpret_cast<const QT*>(a.Q) + ((size_t)(a.q_batched ? bh : h) * M + (m < M ? m : M - 1)) * D;
    };
    const float* qm0 = a.qmul0 ? a.qmul0 + (size_t)h * D : nullptr;
    const float* qm1 = a.qmul1 ? a.qmul1 + (size_t)h * D : nullptr;
    const int m = mg * 32 + li;
    QKOp<bf16, D> qop;
    float qn2;
    const float qerr2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(
        wave_max(load_q_row<D>(qop, nullptr, qrow(), g, a.qscale, a.norm_q != 0, a.eps, qm0, qm1, &qn2)))));
    qn2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(qn2))));
    if (m >= M) zero_op<D>(qop);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    RowSum<D> wsum(lane);
    float kmax2 = 0.f, kerr2 = 0.f;

    const bf16* Xb = pa.X + (size_t)b * N * kProjC;
    bf16* Kw = pa.Kout ? pa.Kout + (size_t)bh * N * D : nullptr;
    __syncthreads();  // the previous piece is done with every LDS tile
    stage_wt<D, NW>(wt, pa.WK + (size_t)h * kProjC * D, pa.WV + (size_t)h * kProjC * D, nm);
    dma_x<NW>(xt, Xb, n_lo, n_hi, wave, lane);
    for (int t0 = n_lo; t0 < n_hi; t0 += ROWS) {
      wait_dma();
      __syncthreads();  // X tile landed, W^T staged; the previous attention is done with the key and value tiles
      project_tile<D, NW>(xt, wt, kt, vt, nm, wave, lane, kerr2);
      __syncthreads();  // key and value tiles complete; the X tile is free
      if constexpr (NK) {
        norm_tile<D, NW>(kt, wave, lane, a.eps);
        __syncthreads();
      }
      kmax2 = tile_key_max<D, NW>(kt, wave, lane, kmax2, Kw ? Kw + (size_t)t0 * D : nullptr, n_hi - t0);
      if (t0 + ROWS < n_hi) dma_x<NW>(xt, Xb, t0 + ROWS, n_hi, wave, lane);
      encode_tile<D, NW, WN, 0>(ka, va, t0 + 32 * ng, n_hi, g, lane, qop, wsum, acc);
    }
    kmax2 = wave_max(kmax2);
    kerr2 = wave_max(kerr2);
    if (lane == 0) { kred[wave] = kmax2; ered[wave] = kerr2; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) { kmax2 = fmaxf(kmax2, kred[w]); kerr2 = fmaxf(kerr2, ered[w]); }
    if (a.part_km && threadIdx.x < WN)  // the norms of the stored keys, for the decode
      a.part_km[(size_t)bhl * a.pmax + slot - ng + threadIdx.x] = kmax2;
    // The fast scores q~ . k~ use rounded queries and rounded projected keys:
    // |q~ . k~ - q . k| <= |q~ - q| |k| + |q| |k~ - k| + |q~ - q| |k~ - k|.
    // Normalised keys are the keys by definition (rounded like stored inputs).
    if (NK) kerr2 = 0.f;
    const float serr = sqrtf(qerr2 * kmax2) + sqrtf(qn2 * kerr2) + sqrtf(qerr2 * kerr2);
    float ltot = wsum.total(li, acc), shift = 0.f;
    const bool redo = serr * serr > kScoreErr2 || fast_failed(ltot, n_lo + 32 * ng < n_hi, acc);
    if (lane == 0) cred[wave] = redo;
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) any = any || cred[w] != 0;
    if (any) {  // workgroup-uniform: every wave projects the tiles again
      QKOp<bf16, D> qhi, qlo;
      f32x16 negs = {}, cacc = {};
      float lsum = 0.f;
      bool started = false;
      if (redo) {
        load_q_row<D>(qhi, &qlo, qrow(), g, a.qscale, a.norm_q != 0, a.eps, qm0, qm1);
        if (m >= M) { zero_op<D>(qhi); zero_op<D>(qlo); }
      }
      for (int t0 = n_lo; t0 < n_hi; t0 += ROWS) {
        __syncthreads();  // the last readers of the X, key and value tiles are done
        dma_x<NW>(xt, Xb, t0, n_hi, wave, lane);
        wait_dma();
        __syncthreads();
        float unused = 0.f;
        project_tile<D, NW>(xt, wt, kt, vt, nm, wave, lane, unused, NK ? nullptr : kl);
        __syncthreads();
        if constexpr (NK) {
          norm_tile<D, NW>(kt, wave, lane, a.eps);
          __syncthreads();
        }
        // with shared keys and values (not normalised) the values keep the
        // rounded keys, as the fast loop uses them
        if (redo) careful_tile_lds<D>(kt, NK ? nullptr : kl, alias ? kt : vt, t0, n_hi, ng, WN, ROWS, lane, qhi, qlo,
                                      negs, started, lsum, cacc);
      }
      if (redo) {
        acc = cacc;
        ltot = pair_sum(lsum);
        shift = -negs[0];
      }
    }
    if (!redo) {  // the fast partial, renormalised to a power-of-two shift
      const int e = __builtin_amdgcn_frexp_expf(ltot);
      const float sc = __builtin_amdgcn_ldexpf(1.f, -e);
      acc = acc * sc;
      ltot *= sc;
      shift = (float)e;
    }
    if (m < M) {
      const size_t p = (size_t)bhl * a.pmax + slot;
      float* dst = a.part_acc + (p * M + m) * D;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (8 * c + 4 * g < D) {
          f32x4 v = {acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
          *reinterpret_cast<f32x4*>(dst + 8 * c + 4 * g) = v;
        }
      }
      if (g == 0) a.part_al[p * M + m] = make_float2(shift, ltot);
    }
    x = hb + n_hi;
  }
}

template <typename QT, int NW, int WN, bool NK>
int launch_proj_k(const ProjArgs& pa, hipStream_t st) {
  return launch(encode_proj_kernel<QT, 32, NW, WN, NK>, dim3(pa.e.nwg), dim3(NW * 64), 0, st, pa);
}

template <typename QT, bool NK>
int launch_proj_w(const ProjArgs& pa, int NW, int WN, hipStream_t st) {
  if (NW == 8 && WN == 1) return launch_proj_k<QT, 8, 1, NK>(pa, st);
  if (NW != 4) return FLARE_ERR_UNSUPPORTED;  // no kernel for this split plan
  if (WN == 4) return launch_proj_k<QT, 4, 4, NK>(pa, st);
  if (WN == 2) return launch_proj_k<QT, 4, 2, NK>(pa, st);
  return launch_proj_k<QT, 4, 1, NK>(pa, st);
}

// The encode of all heads from the block input (bf16, D = 32, C = kProjC);
// qtype is the element type of Q; nm as for launch_encode (norm_k: the
// projected keys are N_0-normalised in LDS, and written so when Kout is set).
int launch_encode_proj(const void* X, const void* WK, const void* WV, bf16* Kout, const void* Q, int qtype,
                       int q_batched, int H, int N, int M, float qscale, float* part_acc, float2* part_al,
                       const EncPlan& p, const Norms& nm, hipStream_t st, float* part_km = nullptr) {
  ProjArgs pa;
  EncArgs& a = pa.e;
  a.Q = Q; a.K = nullptr; a.V = nullptr;
  a.part_acc = part_acc; a.part_al = part_al; a.part_km = part_km;
  a.total = p.total;
  a.q_batched = q_batched; a.v_alias = WK == WV; a.H = H; a.N = N; a.M = M;
  a.G = p.G; a.nwg = p.nwg; a.pmax = p.pmax; a.bh0 = 0;
  a.qscale = qscale;
  a.norm_q = nm.norm_q; a.qmul0 = nm.qmul0; a.qmul1 = nm.qmul1; a.eps = nm.eps;
  pa.X = (const bf16*)X; pa.WK = (const bf16*)WK; pa.WV = (const bf16*)WV; pa.Kout = Kout;
  if (qtype == FLARE_BF16)
    return nm.norm_k ? launch_proj_w<bf16, true>(pa, p.NW, p.WN, st) : launch_proj_w<bf16, false>(pa, p.NW, p.WN, st);
  return nm.norm_k ? launch_proj_w<float, true>(pa, p.NW, p.WN, st) : launch_proj_w<float, false>(pa, p.NW, p.WN, st);
}

}  // namespace
