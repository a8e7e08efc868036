// Decode-shaped GEMM core for the sparse gated FFN on gfx950.
//
// C[n, m] = sum_k A[n, k] B[m, k] with many weight rows n and few tokens m.
// Each wave streams 16-row blocks of A from HBM straight into registers in the
// MFMA operand layout (lane l: row l%16, 8 consecutive k at (l/16)*8, i.e. 64
// contiguous bytes per row per instruction) and multiplies them with 16-token
// blocks of B on v_mfma_f32_16x16x32_bf16. A workgroup of WN x WK waves covers
// NT = 16*RB*WN rows; its K range is split over the WK waves and summed in LDS
// in a fixed order. With ks > 1, ks workgroups split K and each writes its own
// fp32 output slab; the consumer adds the slabs (in order) when it loads them,
// so there is no cross-workgroup synchronisation anywhere.
//
// Epilogues (applied to the fp32 tile in LDS):
//   EPI_TWELL   activation + selection + TwELL pack emitted straight from the
//               accumulator tile; a TwELL tile wider than the workgroup tile
//               gets its slot offsets from the earlier sub-tiles' counts
//               (epoch-tagged 64-bit words). [Sparser/Faster/Lighter page
//               (news.neo-ai.one, "Sparser, Faster, Lighter Transformer
//               Language Models"), section "TwELL 減掉轉換開銷".]
//   EPI_STORE_F32  fp32 store (low-rank intermediate slabs, or g).
//   EPI_WINA    h = a(z) * u and score |h| * c per neuron [WINA page, section 3.1].
//   EPI_DENSE_H hidden h = a(z) * u of the dense evaluation.
//   EPI_Y       output rows, optionally scattered through a token list.
#pragma once
#include <type_traits>

#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

struct TileView {
  const float* t;  // LDS tile, row r (weight row), column m (token slot)
  int ldt, nt, n0, m0, mcnt, rpm;
};

__device__ __forceinline__ int tok_id(const EpiDesc& e, int slot) { return e.tok_of ? e.tok_of[slot] : slot; }
__device__ __forceinline__ float bias_of(const EpiDesc& e, int tok) { return e.bias ? e.bias[tok] : e.bias_scalar; }
__device__ __forceinline__ float cut_of(const EpiDesc& e, int tok) {
  return e.sel == SEL_THRESH ? fmaxf(e.tau[tok], 0.f) : 0.f;
}
__device__ __forceinline__ float act_fn(float z, int act) {
  return act == ACT_RELU ? fmaxf(z, 0.f) : z / (1.f + expf(-z));
}
// Activation value of the dense evaluation with the selection mask applied.
__device__ __forceinline__ float masked_act(const EpiDesc& e, float z, int tok) {
  if (e.sel == SEL_TOPK) return act_fn(z, e.act);
  return z > cut_of(e, tok) ? z : 0.f;
}
__device__ __forceinline__ void store_out(void* base, size_t i, float v, int f32) {
  if (f32) reinterpret_cast<float*>(base)[i] = v;
  else reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)f2bf(v);
}

// ------------------------------------------------------------------ epilogues
__device__ __forceinline__ void epi_store_f32(const EpiDesc& e, const TileView& v, int ksi) {
  float* out = e.out + (size_t)ksi * e.out_slab;
  for (int p = threadIdx.x; p < v.nt * v.mcnt; p += blockDim.x) {
    const int r = p % v.nt, m = p / v.nt;
    out[(size_t)(v.m0 + m) * e.ldo + v.n0 + r] = v.t[r * v.ldt + m];
  }
}

// TwELL emission: the tile covers nt neurons [n0, n0 + nt), sub-tile q of
// TwELL tile j (Q = T / nt). Three block-wide phases, so that the look-back
// costs one memory round for the whole tile rather than one per token:
//   1. one wave per token slot counts the active neurons (ballot + popcount)
//      and publishes the count (epoch-tagged word) when Q > 1;
//   2. every (token, earlier sub-tile) pair is read by one thread, waiting
//      for this pass's epoch, and added into the token's offset in LDS (the
//      words are sub-tile-major, so a wave reads 64 consecutive tokens' words);
//   3. one wave per token slot writes its entries in ascending order at that
//      offset (ballot + prefix popcount), and the last sub-tile writes cnt and
//      the padding.
constexpr int kTwellMaxSlots = 128;
__device__ __forceinline__ void epi_twell(const EpiDesc& e, const TileView& v, uint32_t* ctrl) {
  __shared__ int s_off[kTwellMaxSlots];
  __shared__ float s_bias[kTwellMaxSlots], s_cut[kTwellMaxSlots];
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int Q = e.T / v.nt, q = (v.n0 % e.T) / v.nt, j = v.n0 / e.T;
  const int ntiles = e.F / e.T;
  // pass epoch of the look-back words (advanced by the routing pass after
  // every gate pass); only sub-tiled TwELL tiles need it
  const uint32_t epoch = Q > 1 ? __hip_atomic_load(&ctrl[CTRL_EPOCH], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u : 0u;
  const WaitCtl wc = Q > 1 ? wait_ctl(ctrl, epoch) : WaitCtl{0u, 0u};
  // every token's bias and cut, read in one parallel round
  for (int m = threadIdx.x; m < v.mcnt; m += blockDim.x) {
    s_off[m] = 0;
    s_bias[m] = bias_of(e, v.m0 + m);
    s_cut[m] = cut_of(e, v.m0 + m);
  }
  __syncthreads();
  // phase 1
  for (int m = wave; m < v.mcnt; m += nw) {
    const int tok = v.m0 + m;
    const float b = s_bias[m], cut = s_cut[m];
    int c_local = 0;
    for (int c0 = 0; c0 < v.nt; c0 += 64) {
      const int r = c0 + lane;
      bool act = false;
      if (r < v.nt) {
        const float gv = v.t[r * v.ldt + m];
        if (e.g_debug) e.g_debug[(size_t)tok * e.F + v.n0 + r] = gv;
        act = (gv + b) > cut;
      }
      c_local += __popcll(ballot64(act));
    }
    if (Q > 1 && lane == 0)
      store64_relaxed(e.lb + ((size_t)j * Q + q) * e.lb_ld + tok, ((uint64_t)epoch << 32) | (uint32_t)c_local);
  }
  __syncthreads();
  // phase 2
  if (Q > 1 && q > 0) {
    for (int p = threadIdx.x; p < v.mcnt * q; p += blockDim.x) {
      const int pp = p / v.mcnt, m = p - pp * v.mcnt;   // consecutive threads: consecutive tokens
      const uint64_t* wp = e.lb + ((size_t)j * Q + pp) * e.lb_ld + v.m0 + m;
      atomicAdd(&s_off[m], (int)tagged_wait(wp, load64_relaxed(wp), wc, ctrl));
    }
  }
  __syncthreads();
  // phase 3
  for (int m = wave; m < v.mcnt; m += nw) {
    const int tok = v.m0 + m;
    const float b = s_bias[m], cut = s_cut[m];
    int run = s_off[m];
    const size_t slot0 = ((size_t)tok * ntiles + j) * e.E;
    for (int c0 = 0; c0 < v.nt; c0 += 64) {
      const int r = c0 + lane;
      float z = 0.f;
      bool act = false;
      if (r < v.nt) {
        z = v.t[r * v.ldt + m] + b;
        act = z > cut;
      }
      const uint64_t bal = ballot64(act);
      const int pos = run + __popcll(bal & lanemask_lt());
      if (act && pos < e.E) {
        e.idx[slot0 + pos] = (uint16_t)(q * v.nt + r);
        store_out(e.val, slot0 + pos, z, e.out_f32);
      }
      run += __popcll(bal);
    }
    if (q == Q - 1) {
      if (lane == 0) e.cnt[(size_t)tok * ntiles + j] = run;
      for (int s = min(run, e.E) + lane; s < e.E; s += 64) {
        e.idx[slot0 + s] = 0xFFFF;
        store_out(e.val, slot0 + s, 0.f, e.out_f32);
      }
    }
  }
  __syncthreads();                                  // s_off is reused by the next call
}

// rows [0, rpm) of the tile are the gate, [rpm, 2 rpm) the up projection of
// the same neurons [n0, n0 + rpm).
__device__ __forceinline__ void epi_wina(const EpiDesc& e, const TileView& v) {
  for (int p = threadIdx.x; p < v.rpm * v.mcnt; p += blockDim.x) {
    const int r = p % v.rpm, m = p / v.rpm;
    const int tok = v.m0 + m, n = v.n0 + r;
    const float gv = v.t[r * v.ldt + m], uv = v.t[(v.rpm + r) * v.ldt + m];
    const float h = act_fn(gv + bias_of(e, tok), e.act) * uv;
    const float s = fabsf(h) * e.colnorm[n];
    const size_t o = (size_t)tok * e.F + n;
    e.s_buf[o] = s;
    e.h_buf[o] = h;
    if (e.g_debug) e.g_debug[o] = gv;
    if (e.s_debug) e.s_debug[o] = s;
  }
}

// Hidden activations of the dense evaluation. Two-matrix tiles carry the gate
// and up rows; one-matrix tiles carry up rows and read the gate from g_ext.
template <int NMAT>
__device__ __forceinline__ void epi_dense_h(const EpiDesc& e, const TileView& v) {
  for (int p = threadIdx.x; p < v.rpm * v.mcnt; p += blockDim.x) {
    const int r = p % v.rpm, m = p / v.rpm;
    const int slot = v.m0 + m, tok = tok_id(e, slot), n = v.n0 + r;
    float gv, uv;
    if (NMAT == 2) {
      gv = v.t[r * v.ldt + m];
      uv = v.t[(v.rpm + r) * v.ldt + m];
      if (e.g_debug) e.g_debug[(size_t)slot * e.F + n] = gv;   // the gate values, for a pack built from them
    } else {
      gv = e.g_ext[(size_t)slot * e.F + n];
      uv = v.t[r * v.ldt + m];
    }
    const float h = masked_act(e, gv + bias_of(e, tok), tok) * uv;
    store_out(e.hout, (size_t)slot * e.ldh + n, h, e.out_f32);
  }
}

__device__ __forceinline__ void epi_y(const EpiDesc& e, const TileView& v) {
  for (int p = threadIdx.x; p < v.nt * v.mcnt; p += blockDim.x) {
    const int r = p % v.nt, m = p / v.nt;
    const int row = e.yrows ? e.yrows[v.m0 + m] : v.m0 + m;
    store_out(e.y, (size_t)row * e.ldy + v.n0 + r, v.t[r * v.ldt + m], e.out_f32);
  }
}

template <int NMAT, int EPI>
__device__ __forceinline__ void run_epilogue(const EpiDesc& e, const TileView& v, uint32_t* ctrl, int ksi) {
  if (EPI == EPI_STORE_F32) epi_store_f32(e, v, ksi);
  if (EPI == EPI_WINA) epi_wina(e, v);
  if (EPI == EPI_DENSE_H) epi_dense_h<NMAT>(e, v);
  if (EPI == EPI_Y) epi_y(e, v);
  if (EPI == EPI_TWELL) epi_twell(e, v, ctrl);
}

// Low-rank gate: the workgroups of weight tile 0 also store the summed
// intermediate t (from the first stage's slabs) for later consumers.
__device__ __forceinline__ void store_summed_t(const GemmDesc& g, const EpiDesc& e, int m0, int mcnt) {
  const float* B = reinterpret_cast<const float*>(g.B);
  for (int p = threadIdx.x; p < mcnt * g.K; p += blockDim.x) {
    const int m = p / g.K, k = p % g.K;
    const size_t o = (size_t)(m0 + m) * g.ldb + k;
    float s = B[o];
    for (int q = 1; q < g.b_nsum; ++q) s += B[o + (size_t)q * g.b_slab];
    e.t_out[(size_t)(m0 + m) * g.K + k] = s;
  }
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int RB, int MB, int BM, int U>
struct Frags {
  uint4 a[U][RB];
  uint4 b[U][MB][BM == B_F32_SPLIT ? 2 : 1];
};

// U: k-chunks whose loads are all issued before the MFMAs that use them
// (one memory round trip per U chunks), bounded by the fragment registers.
template <int RB, int MB, int BM>
struct UnrollOf {
  static constexpr int NB = BM == B_F32_SPLIT ? 2 : 1;
  static constexpr int W = RB + MB * NB;
  static constexpr int value = W <= 3 ? 8 : (W <= 5 ? 4 : 2);
};

template <int RB, int WN, int WK, int MB, int BM, int NMAT, int EPI, int NSUM>
__global__ __launch_bounds__(64 * WN * WK) void k_gemm_bf16(const GemmDesc g, const EpiDesc e) {
  constexpr int NT = 16 * RB * WN, MT = 16 * MB, LDT = MT + 1, RPM = NT / NMAT;
  constexpr int U = UnrollOf<RB, MB, BM>::value;
  __shared__ float tile[NT * LDT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int tile_id = blockIdx.x / g.ks, ksi = blockIdx.x % g.ks;
  const int m0 = blockIdx.y * MT;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;
  const int mcnt = min(MT, Mtot - m0);
  const int n0 = tile_id * RPM;

  const int kct = g.K >> 5;
  const int per_ks = (kct + g.ks - 1) / g.ks;
  const int kc0 = min(kct, ksi * per_ks), kc1 = min(kct, kc0 + per_ks);
  const int per_w = (kc1 - kc0 + WK - 1) / WK;
  const int kw0 = min(kc1, kc0 + wk * per_w), kw1 = min(kc1, kw0 + per_w);

  const uint16_t* ap[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (wn * RB + rb) * 16 + (lane & 15);
    const int mat = r / RPM, rr = n0 + (r % RPM);
    ap[rb] = reinterpret_cast<const uint16_t*>(mat ? g.A1 : g.A0) + (size_t)rr * g.lda + (lane >> 4) * 8;
  }
  constexpr int BES = (BM == B_F32_SPLIT) ? 4 : 2;
  const char* bp[MB];
  bool bv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + (lane & 15);
    bv[mb] = m < mcnt;
    const int row = bv[mb] ? (g.gather ? g.gather[m0 + m] : m0 + m) : 0;
    bp[mb] = reinterpret_cast<const char*>(g.B) + ((size_t)row * g.ldb + (lane >> 4) * 8) * BES;
  }
  const size_t slab_bytes = (size_t)g.b_slab * 4;

  f32x4_t acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto body = [&](int kc, auto uu) {
    constexpr int UU = decltype(uu)::value;
    Frags<RB, MB, BM, UU> f;
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) f.a[u][rb] = ldg16(ap[rb] + (size_t)(kc + u) * 32);
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (BM == B_F32_SPLIT) {
          const char* p = bp[mb] + (size_t)(kc + u) * 32 * 4;
          uint4 v0 = uint4{0, 0, 0, 0}, v1 = uint4{0, 0, 0, 0};
          if (bv[mb]) {
            v0 = ldg16(p);
            v1 = ldg16(p + 16);
#pragma unroll
            for (int q = 1; q < NSUM; ++q) {            // ordered sum of the producer's slabs
              const uint4 w0 = ldg16(p + q * slab_bytes), w1 = ldg16(p + q * slab_bytes + 16);
              v0.x = __float_as_uint(__uint_as_float(v0.x) + __uint_as_float(w0.x));
              v0.y = __float_as_uint(__uint_as_float(v0.y) + __uint_as_float(w0.y));
              v0.z = __float_as_uint(__uint_as_float(v0.z) + __uint_as_float(w0.z));
              v0.w = __float_as_uint(__uint_as_float(v0.w) + __uint_as_float(w0.w));
              v1.x = __float_as_uint(__uint_as_float(v1.x) + __uint_as_float(w1.x));
              v1.y = __float_as_uint(__uint_as_float(v1.y) + __uint_as_float(w1.y));
              v1.z = __float_as_uint(__uint_as_float(v1.z) + __uint_as_float(w1.z));
              v1.w = __float_as_uint(__uint_as_float(v1.w) + __uint_as_float(w1.w));
            }
          }
          f.b[u][mb][0] = v0;
          f.b[u][mb][BM == B_F32_SPLIT ? 1 : 0] = v1;
        } else {
          const char* p = bp[mb] + (size_t)(kc + u) * 32 * 2;
          f.b[u][mb][0] = bv[mb] ? ldg16(p) : uint4{0, 0, 0, 0};
        }
      }
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (BM == B_F32_SPLIT) {
          // t = hi + lo with hi = bf16(t), lo = bf16(t - hi): two exact-product MFMAs
          const uint4 p0 = f.b[u][mb][0], p1 = f.b[u][mb][BM == B_F32_SPLIT ? 1 : 0];
          const float x[8] = {__uint_as_float(p0.x), __uint_as_float(p0.y), __uint_as_float(p0.z),
                              __uint_as_float(p0.w), __uint_as_float(p1.x), __uint_as_float(p1.y),
                              __uint_as_float(p1.z), __uint_as_float(p1.w)};
          uint32_t hi[8], lo[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            hi[q] = f2bf(x[q]);
            lo[q] = f2bf(x[q] - bf2f(hi[q]));
          }
          const uint4 bh = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
          const uint4 bl = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.a[u][rb]), as_bf16x8(bh), acc[rb][mb], 0, 0, 0);
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.a[u][rb]), as_bf16x8(bl), acc[rb][mb], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.a[u][rb]), as_bf16x8(f.b[u][mb][0]), acc[rb][mb], 0, 0, 0);
        }
      }
  };
  int kc = kw0;
  for (; kc + U <= kw1; kc += U) body(kc, std::integral_constant<int, U>{});
  for (; kc < kw1; ++kc) body(kc, std::integral_constant<int, 1>{});

  // fixed-order reduction of the K-split waves into the LDS tile
  for (int s = 0; s < WK; ++s) {
    if (wk == s) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const int row = (wn * RB + rb) * 16 + 4 * (lane >> 4) + vv;
            const int col = mb * 16 + (lane & 15);
            float* p = &tile[row * LDT + col];
            if (s == 0) *p = acc[rb][mb][vv];
            else *p += acc[rb][mb][vv];
          }
    }
    __syncthreads();
  }
  if (EPI == EPI_TWELL && BM == B_F32_SPLIT && e.t_out && tile_id == 0) store_summed_t(g, e, m0, mcnt);
  const TileView v{tile, LDT, NT, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(e, v, g.ctrl, ksi);
}

// ------------------------------------------------------------------ decode GEMV (VALU)
// For a few tokens (M <= 8) and K <= 4096 the contraction is a batch of dot
// products: a wave reads weight rows in 1 KB pieces (64 lanes x 16 B, fully
// contiguous), multiplies them with the tokens' matching 8 elements held in
// registers (loaded once per wave), and reduces each (row, token) across the
// wave. Rows per workgroup need not be a multiple of 16, so small matrices
// still spread over enough workgroups. Eight 1 KB loads are in flight per wave.
// The result goes through the same LDS tile and epilogues as the MFMA kernel.
template <int NW, int MAXM, int NKC, bool BF32, int NMAT, int EPI>
__global__ __launch_bounds__(64 * NW) void k_gemv_bf16(const GemmDesc g, const EpiDesc e) {
  constexpr int MT = 16, LDT = MT + 1;
  constexpr int BW = BF32 ? 2 : 1;                // uint4 per token per piece
  constexpr int RPG = 8 / NKC;                    // rows per group of 8 pieces
  __shared__ float tile[128 * LDT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NT = g.nt, RPM = NT / NMAT;
  const int tile_id = blockIdx.x;
  const int m0 = blockIdx.y * MT;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;
  const int mcnt = min(MAXM, Mtot - m0);
  const int n0 = tile_id * RPM;
  const int nkc = (g.K + 511) / 512;              // pieces per row (<= NKC); the last may be partial
  // does this lane's 8-element slice of piece c exist?
  auto lane_in = [&](int c) { return c < nkc && c * 512 + lane * 8 < g.K; };

  // tokens' inputs for this lane: piece c, elements [c*512 + lane*8, +8)
  uint4 bx[NKC][MAXM][BW];
#pragma unroll
  for (int c = 0; c < NKC; ++c)
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
#pragma unroll
      for (int w = 0; w < BW; ++w) {
        bx[c][m][w] = uint4{0, 0, 0, 0};
        if (m < mcnt && lane_in(c)) {
          const int row = g.gather ? g.gather[m0 + m] : m0 + m;
          const char* p = reinterpret_cast<const char*>(g.B) +
                          ((size_t)row * g.ldb + (size_t)c * 512 + lane * 8) * (BF32 ? 4 : 2) + w * 16;
          bx[c][m][w] = ldg16(p);
        }
      }

  const int rpw = (NT + NW - 1) / NW;            // rows of this wave: wave, wave + NW, ...
  for (int rl0 = 0; rl0 < rpw; rl0 += RPG) {
    uint4 a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rl = rl0 + q / NKC, c = q % NKC;
      const int r = wave + rl * NW;
      a[q] = uint4{0, 0, 0, 0};
      if (rl < rpw && r < NT && lane_in(c)) {
        const int mat = r / RPM, rr = n0 + (r % RPM);
        a[q] = ldg16(reinterpret_cast<const uint16_t*>(mat ? g.A1 : g.A0) + (size_t)rr * g.lda + (size_t)c * 512 + lane * 8);
      }
    }
    float acc[RPG][MAXM];
#pragma unroll
    for (int q = 0; q < RPG; ++q)
#pragma unroll
      for (int m = 0; m < MAXM; ++m) acc[q][m] = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      constexpr int dummy = 0;
      (void)dummy;
      float f[8];
      unpack8(a[q], f);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float xv[8];
        const uint4 b0 = bx[q % NKC][m][0];
        if (BF32) {
          const uint4 b1 = bx[q % NKC][m][BW - 1];
          xv[0] = __uint_as_float(b0.x); xv[1] = __uint_as_float(b0.y); xv[2] = __uint_as_float(b0.z); xv[3] = __uint_as_float(b0.w);
          xv[4] = __uint_as_float(b1.x); xv[5] = __uint_as_float(b1.y); xv[6] = __uint_as_float(b1.z); xv[7] = __uint_as_float(b1.w);
        } else {
          unpack8(b0, xv);
        }
        float sacc = acc[q / NKC][m];
#pragma unroll
        for (int k = 0; k < 8; ++k) sacc = fmaf(f[k], xv[k], sacc);
        acc[q / NKC][m] = sacc;
      }
    }
#pragma unroll
    for (int q = 0; q < RPG; ++q) {
      const int rl = rl0 + q, r = wave + rl * NW;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const float v = wave_sum(acc[q][m]);
        if (lane == m && r < NT && rl < rpw) tile[r * LDT + m] = v;
      }
    }
  }
  __syncthreads();
  if (EPI == EPI_TWELL && BF32 && e.t_out && tile_id == 0) store_summed_t(g, e, m0, mcnt);
  const TileView v{tile, LDT, NT, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(e, v, g.ctrl, 0);
}

// registers held for the tokens' inputs: NKC * MAXM * BW uint4 (<= 32)
template <int NW, int MAXM, int NKC, bool BF32, int NMAT, int EPI>
static hipError_t go_gemv_1(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  if constexpr (NKC * MAXM * (BF32 ? 2 : 1) > 32) {
    return hipErrorInvalidValue;
  } else {
    ffn_launch((k_gemv_bf16<NW, MAXM, NKC, BF32, NMAT, EPI>), grid, dim3(64 * NW), 0, s, g, e);
    return hipGetLastError();
  }
}

template <int NW, int NKC, bool BF32, int NMAT, int EPI>
static hipError_t go_gemv_m(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  if (g.M <= 1) return go_gemv_1<NW, 1, NKC, BF32, NMAT, EPI>(g, e, grid, s);
  if (g.M <= 4) return go_gemv_1<NW, 4, NKC, BF32, NMAT, EPI>(g, e, grid, s);
  return go_gemv_1<NW, 8, NKC, BF32, NMAT, EPI>(g, e, grid, s);
}

template <int NW, bool BF32, int NMAT, int EPI>
static hipError_t go_gemv_k(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  const int nkc = (g.K + 511) / 512;
  if (BF32) return nkc == 1 ? go_gemv_m<NW, 1, BF32, NMAT, EPI>(g, e, grid, s) : hipErrorInvalidValue;
  if (nkc == 1) return go_gemv_m<NW, 1, BF32, NMAT, EPI>(g, e, grid, s);
  if (nkc == 2) return go_gemv_m<NW, 2, BF32, NMAT, EPI>(g, e, grid, s);
  if (nkc <= 4) return go_gemv_m<NW, 4, BF32, NMAT, EPI>(g, e, grid, s);
  if (nkc <= 8) return go_gemv_m<NW, 8, BF32, NMAT, EPI>(g, e, grid, s);
  return hipErrorInvalidValue;
}

// decode GEMV dispatch: 4 or 16 waves per workgroup; B bf16, or fp32 (K <= 512)
template <int NMAT, int EPI>
static hipError_t go_gemv(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  const bool bf32 = g.bmode == B_F32_SPLIT;
  if (g.nwaves == 16) return bf32 ? go_gemv_k<16, true, NMAT, EPI>(g, e, grid, s) : go_gemv_k<16, false, NMAT, EPI>(g, e, grid, s);
  if (g.nwaves == 4) return bf32 ? go_gemv_k<4, true, NMAT, EPI>(g, e, grid, s) : go_gemv_k<4, false, NMAT, EPI>(g, e, grid, s);
  return hipErrorInvalidValue;
}

// Whether the decode GEMV handles this shape (host side). The tokens' inputs
// live in NKC * MAXM * BW uint4 registers per lane: at most 8 of them in
// 16-wave workgroups (128 VGPRs per lane), 32 in 4-wave ones; larger inputs
// would spill, and the MFMA kernel takes those shapes.
inline bool gemv_ok(const GemmDesc& g) {
  if (g.dtype != DT_BF16 || g.M > 8 || g.ks != 1 || g.nt > 128 || g.b_nsum != 1) return false;
  const int nkc = (g.K + 511) / 512;
  const int kc = nkc <= 1 ? 1 : (nkc <= 2 ? 2 : (nkc <= 4 ? 4 : 8));
  if (nkc > 8) return false;
  const int mx = g.M <= 1 ? 1 : (g.M <= 4 ? 4 : 8);
  const int bw = g.bmode == B_F32_SPLIT ? 2 : 1;
  if (bw == 2 && nkc != 1) return false;
  return kc * mx * bw <= (g.nwaves == 16 ? 8 : 32);
}

// ------------------------------------------------------------------ fp32 VALU kernel
// fp32 configurations are small; one thread per (row, token) dot product, k
// ascending with fused multiply-adds; B may be a sum of slabs.
template <int NT, int NMAT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(const GemmDesc g, const EpiDesc e) {
  constexpr int MT = 16, LDT = MT + 1, RPM = NT / NMAT;
  __shared__ float tile[NT * LDT];
  const int tile_id = blockIdx.x / g.ks, ksi = blockIdx.x % g.ks;
  const int m0 = blockIdx.y * MT;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;
  const int mcnt = min(MT, Mtot - m0);
  const int n0 = tile_id * RPM;
  const int kct = g.K / 4;
  const int per_ks = (kct + g.ks - 1) / g.ks;
  const int k0 = min(kct, ksi * per_ks) * 4, k1 = min(kct, ksi * per_ks + per_ks) * 4;
  for (int p = threadIdx.x; p < NT * mcnt; p += blockDim.x) {
    const int r = p % NT, m = p / NT;
    const int mat = r / RPM, rr = n0 + (r % RPM);
    const float* a = reinterpret_cast<const float*>(mat ? g.A1 : g.A0) + (size_t)rr * g.lda;
    const int row = g.gather ? g.gather[m0 + m] : m0 + m;
    const float* b = reinterpret_cast<const float*>(g.B) + (size_t)row * g.ldb;
    float s = 0.f;
    for (int k = k0; k < k1; k += 4) {
      const float4 av = *reinterpret_cast<const float4*>(a + k);
      float4 bw = *reinterpret_cast<const float4*>(b + k);
      for (int q = 1; q < g.b_nsum; ++q) {
        const float4 w = *reinterpret_cast<const float4*>(b + k + (size_t)q * g.b_slab);
        bw.x += w.x; bw.y += w.y; bw.z += w.z; bw.w += w.w;
      }
      s = fmaf(av.x, bw.x, s);
      s = fmaf(av.y, bw.y, s);
      s = fmaf(av.z, bw.z, s);
      s = fmaf(av.w, bw.w, s);
    }
    tile[r * LDT + m] = s;
  }
  __syncthreads();
  if (EPI == EPI_TWELL && e.t_out && tile_id == 0) store_summed_t(g, e, m0, mcnt);
  const TileView v{tile, LDT, NT, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(e, v, g.ctrl, ksi);
}

// ------------------------------------------------------------------ dispatch helpers
template <int RB, int WN, int WK, int MB, int BM, int NMAT, int EPI>
static hipError_t go_bf16(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  const dim3 blk(64 * WN * WK);
  if (BM == B_F32_SPLIT) {
    switch (g.b_nsum) {
      case 1: ffn_launch((k_gemm_bf16<RB, WN, WK, MB, BM, NMAT, EPI, 1>), grid, blk, 0, s, g, e); break;
      case 2: ffn_launch((k_gemm_bf16<RB, WN, WK, MB, BM, NMAT, EPI, 2>), grid, blk, 0, s, g, e); break;
      case 4: ffn_launch((k_gemm_bf16<RB, WN, WK, MB, BM, NMAT, EPI, 4>), grid, blk, 0, s, g, e); break;
      case 8: ffn_launch((k_gemm_bf16<RB, WN, WK, MB, BM, NMAT, EPI, 8>), grid, blk, 0, s, g, e); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (g.b_nsum != 1) return hipErrorInvalidValue;
    ffn_launch((k_gemm_bf16<RB, WN, WK, MB, BM, NMAT, EPI, 1>), grid, blk, 0, s, g, e);
  }
  return hipGetLastError();
}

template <int RB, int WN, int WK, int BM, int NMAT, int EPI>
static hipError_t pick_mb(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  switch (g.mt) {
    case 16: return go_bf16<RB, WN, WK, 1, BM, NMAT, EPI>(g, e, grid, s);
    case 32: return go_bf16<RB, WN, WK, 2, BM, NMAT, EPI>(g, e, grid, s);
    case 64: return go_bf16<RB, WN, WK, 4, BM, NMAT, EPI>(g, e, grid, s);
  }
  return hipErrorInvalidValue;
}

// nt / nwaves -> (RB, WN, WK); two-matrix tiles need at least 32 rows
template <int BM, int NMAT, int EPI>
static hipError_t pick_shape(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  if (g.nwaves == 16) {
    switch (g.nt) {
      case 16: if (NMAT == 1) return pick_mb<1, 1, 16, BM, NMAT, EPI>(g, e, grid, s); break;
      case 32: return pick_mb<1, 2, 8, BM, NMAT, EPI>(g, e, grid, s);
      case 64: return pick_mb<1, 4, 4, BM, NMAT, EPI>(g, e, grid, s);
      case 128: return pick_mb<1, 8, 2, BM, NMAT, EPI>(g, e, grid, s);
    }
    return hipErrorInvalidValue;
  }
  switch (g.nt) {
    case 16: if (NMAT == 1) return pick_mb<1, 1, 4, BM, NMAT, EPI>(g, e, grid, s); break;
    case 32: return pick_mb<1, 2, 2, BM, NMAT, EPI>(g, e, grid, s);
    case 64: return pick_mb<1, 4, 1, BM, NMAT, EPI>(g, e, grid, s);
    case 128: return pick_mb<2, 4, 1, BM, NMAT, EPI>(g, e, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int NMAT, int EPI>
static hipError_t go_f32(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  switch (g.nt) {
    case 16: if (NMAT == 1) { ffn_launch((k_gemm_f32<16, NMAT, EPI>), grid, dim3(256), 0, s, g, e); return hipGetLastError(); } break;
    case 32: ffn_launch((k_gemm_f32<32, NMAT, EPI>), grid, dim3(256), 0, s, g, e); return hipGetLastError();
    case 64: ffn_launch((k_gemm_f32<64, NMAT, EPI>), grid, dim3(256), 0, s, g, e); return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

inline dim3 gemm_grid(const GemmDesc& g) {
  if (g.gemv) return dim3(g.nrows * g.nmat / g.nt, (g.M + 15) / 16);
  const int tiles = g.nrows * g.nmat / g.nt;
  return dim3(tiles * g.ks, (g.M + g.mt - 1) / g.mt);
}

// prefill-shaped GEMM (k_prefill.hip): 128 x 128 LDS-staged MFMA tiles for M >= 128
bool pf_ok(const GemmDesc& g, const EpiDesc& e);
hipError_t launch_gemm_pf(const GemmDesc& g, const EpiDesc& e, hipStream_t s);

// skinny GEMM (k_skinny.hip): 16..64-token blocks, the token tile in LDS
bool sk_ok(const GemmDesc& g, const EpiDesc& e);
hipError_t launch_gemm_sk(const GemmDesc& g, const EpiDesc& e, hipStream_t s);

// entry points per epilogue group (each in its own translation unit)
hipError_t launch_gemm_pack(const GemmDesc& g, const EpiDesc& e, hipStream_t s);    // STORE_F32, TWELL
hipError_t launch_gemm_dense(const GemmDesc& g, const EpiDesc& e, hipStream_t s);   // WINA, DENSE_H, Y

}  // namespace ffn
