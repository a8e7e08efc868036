// Gate / projection GEMMs for decode-sized token counts, with the fused
// epilogues of the sparse FFN:
//   EPI_TWELL   activation + selection + TwELL pack emitted straight from the
//               accumulator tile (no dense activation buffer, no conversion
//               pass), look-back across the sub-tiles of one TwELL tile, and a
//               last-workgroup pass that routes tokens and builds the sparse
//               schedule.  [Sparser/Faster/Lighter page (news.neo-ai.one,
//               "Sparser, Faster, Lighter Transformer Language Models"),
//               sections "TwELL 減掉轉換開銷" and "Hybrid 應對非均勻稀疏".]
//   EPI_STORE_F32  plain fp32 store (low-rank intermediate t = V x, or g).
//   EPI_WINA    h = a(z) * u and score |h| * c for every neuron. [WINA page,
//               section 3.1.]
//   EPI_DENSE_H hidden h = a(z) * u of the dense evaluation (bf16/fp32 out).
//   EPI_Y       output rows (optionally scattered through a token list).
//
// Shape of the problem: C[n, m] = sum_k A[n, k] B[m, k] with many weight rows
// n and few tokens m. Each wave streams 16-row blocks of A from HBM straight
// into registers in the MFMA operand layout (lane l: row l%16, 8 consecutive
// k at (l/16)*8 -- 64 contiguous bytes per row per instruction) and multiplies
// them with 16-token blocks of B on v_mfma_f32_16x16x32_bf16. The K range of a
// workgroup is split over its waves and, for short-N matrices, over ks
// workgroups; partial tiles are summed in a fixed order, so results are
// bit-reproducible run to run.
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
__device__ void epi_store_f32(const EpiDesc& e, const TileView& v) {
  for (int p = threadIdx.x; p < v.nt * v.mcnt; p += blockDim.x) {
    const int r = p % v.nt, m = p / v.nt;
    e.out[(size_t)(v.m0 + m) * e.ldo + v.n0 + r] = v.t[r * v.ldt + m];
  }
}

// TwELL emission. One wave per token slot; the tile covers nt neurons
// [n0, n0 + nt), sub-tile q of TwELL tile j (Q = T / nt sub-tiles). Active
// neurons are compacted in ascending order with a ballot + prefix popcount.
// Sub-tiles learn their starting slot from the earlier sub-tiles' counts,
// published as 64-bit words tagged with the pass epoch (no reset needed).
__device__ void epi_twell(const EpiDesc& e, const TileView& v, uint32_t epoch) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int Q = e.T / v.nt, q = (v.n0 % e.T) / v.nt, j = v.n0 / e.T;
  const int ntiles = e.F / e.T, nsub = e.F / v.nt;
  for (int m = wave; m < v.mcnt; m += nw) {
    const int tok = v.m0 + m;
    const float b = bias_of(e, tok), cut = cut_of(e, tok);
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
    int P = 0;
    if (Q > 1) {
      uint64_t* words = e.lb + (size_t)tok * nsub + (size_t)j * Q;
      if (lane == 0) store64_relaxed(words + q, ((uint64_t)epoch << 32) | (uint32_t)c_local);
      int pv = 0;
      if (lane < q) {
        uint64_t w;
        while (((w = load64_relaxed(words + lane)) >> 32) != epoch) __builtin_amdgcn_s_sleep(1);
        pv = (int)(uint32_t)w;
      }
      P = wave_sum_i(pv);
    }
    int run = P;
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
}

// Routing and the sparse schedule, run by the last workgroup of the gate
// pass: route_t = any tile with cnt > E; dense_list = routed ids ascending;
// offs = exclusive prefix of entry counts over non-routed tokens.
__device__ void twell_finalize(const EpiDesc& e, int M) {
  __shared__ int s_over[1024];
  __shared__ int s_sum[1024];
  __shared__ int s_scan[4];
  const int ntiles = e.F / e.T;
  int base_dense = 0, base_off = 0;
  for (int c0 = 0; c0 < M; c0 += 1024) {
    const int n = min(1024, M - c0);
    for (int i = threadIdx.x; i < 1024; i += blockDim.x) { s_over[i] = 0; s_sum[i] = 0; }
    __syncthreads();
    for (int p = threadIdx.x; p < n * ntiles; p += blockDim.x) {
      const int t = p / ntiles;
      const int c = e.cnt[(size_t)(c0 + t) * ntiles + (p % ntiles)];
      if (c > e.E) atomicOr(&s_over[t], 1);
      atomicAdd(&s_sum[t], c);
    }
    __syncthreads();
    int o[4], cn[4], ro = 0, rn = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = threadIdx.x * 4 + i;
      o[i] = t < n ? s_over[t] : 0;
      cn[i] = (t < n && !o[i]) ? s_sum[t] : 0;
      ro += o[i];
      rn += cn[i];
    }
    int tot_o, tot_n;
    int xo = block_excl_scan<256>(ro, s_scan, &tot_o);
    int xn = block_excl_scan<256>(rn, s_scan, &tot_n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = threadIdx.x * 4 + i;
      if (t < n) {
        const int tok = c0 + t;
        e.route[tok] = (uint8_t)o[i];
        if (o[i]) e.dense_list[base_dense + xo] = tok;
        e.offs[tok] = base_off + xn;
        xo += o[i];
        xn += cn[i];
      }
    }
    base_dense += tot_o;
    base_off += tot_n;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *e.n_dense = base_dense;
    e.offs[M] = base_off;
  }
}

// rows [0, rpm) of the tile are the gate, [rpm, 2 rpm) the up projection of
// the same neurons [n0, n0 + rpm).
__device__ void epi_wina(const EpiDesc& e, const TileView& v) {
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
__device__ void epi_dense_h(const EpiDesc& e, const TileView& v) {
  for (int p = threadIdx.x; p < v.rpm * v.mcnt; p += blockDim.x) {
    const int r = p % v.rpm, m = p / v.rpm;
    const int slot = v.m0 + m, tok = tok_id(e, slot), n = v.n0 + r;
    float gv, uv;
    if (NMAT == 2) {
      gv = v.t[r * v.ldt + m];
      uv = v.t[(v.rpm + r) * v.ldt + m];
    } else {
      gv = e.g_ext[(size_t)slot * e.F + n];
      uv = v.t[r * v.ldt + m];
    }
    const float h = masked_act(e, gv + bias_of(e, tok), tok) * uv;
    store_out(e.hout, (size_t)slot * e.ldh + n, h, e.out_f32);
  }
}

__device__ void epi_y(const EpiDesc& e, const TileView& v) {
  for (int p = threadIdx.x; p < v.nt * v.mcnt; p += blockDim.x) {
    const int r = p % v.nt, m = p / v.nt;
    const int row = e.yrows ? e.yrows[v.m0 + m] : v.m0 + m;
    store_out(e.y, (size_t)row * e.ldy + v.n0 + r, v.t[r * v.ldt + m], e.out_f32);
  }
}

template <int NMAT, int EPI>
__device__ __forceinline__ void run_epilogue(const GemmDesc& g, const EpiDesc& e, const TileView& v,
                                             uint32_t epoch, int Mtot, int* s_flag) {
  if (EPI == EPI_STORE_F32) epi_store_f32(e, v);
  if (EPI == EPI_WINA) epi_wina(e, v);
  if (EPI == EPI_DENSE_H) epi_dense_h<NMAT>(e, v);
  if (EPI == EPI_Y) epi_y(e, v);
  if (EPI == EPI_TWELL) {
    epi_twell(e, v, epoch);
    const uint32_t total = (gridDim.x / g.ks) * gridDim.y;
    if (block_last_arrival(&g.ctrl[CTRL_GATE_DONE], total, s_flag)) {
      twell_finalize(e, Mtot);
      __syncthreads();
      if (threadIdx.x == 0) atomic_store_agent(&g.ctrl[CTRL_EPOCH], epoch);
    }
  }
}

// Sums the ks partial tiles of this (tile, token block) in a fixed order.
// Returns false in every workgroup but the last to arrive.
template <int NT, int MT, int LDT>
__device__ bool splitk_combine(const GemmDesc& g, float* tile, int tile_id, int ksi, int* s_flag) {
  const int tl = blockIdx.y * (gridDim.x / g.ks) + tile_id;
  float* base = g.partial + (size_t)tl * g.ks * NT * MT;
  for (int p = threadIdx.x; p < NT * MT; p += blockDim.x)
    base[(size_t)ksi * NT * MT + p] = tile[(p / MT) * LDT + (p % MT)];
  if (!block_last_arrival(&g.tickets[tl], (uint32_t)g.ks, s_flag)) return false;
  for (int p = threadIdx.x; p < NT * MT; p += blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < g.ks; ++k) s += base[(size_t)k * NT * MT + p];
    tile[(p / MT) * LDT + (p % MT)] = s;
  }
  __syncthreads();
  return true;
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int RB, int MB, int BM, int U>
struct Frags {
  uint4 a[U][RB];
  uint4 b[U][MB][BM == B_F32_SPLIT ? 2 : 1];
};

template <int RB, int WN, int MB, int BM, int NMAT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_bf16(const GemmDesc g, const EpiDesc e) {
  constexpr int WK = 4 / WN, NT = 16 * RB * WN, MT = 16 * MB, LDT = MT + 1, RPM = NT / NMAT;
  constexpr int U = (BM == B_F32_SPLIT && MB >= 2) ? 2 : 4;
  __shared__ float tile[NT * LDT];
  __shared__ int s_flag;
  __shared__ uint32_t s_epoch;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int tile_id = blockIdx.x / g.ks, ksi = blockIdx.x % g.ks;
  const int m0 = blockIdx.y * MT;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;
  const int mcnt = min(MT, Mtot - m0);
  const int n0 = tile_id * RPM;
  if (EPI == EPI_TWELL && threadIdx.x == 0) s_epoch = atomic_load_agent(&g.ctrl[CTRL_EPOCH]) + 1u;

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
          f.b[u][mb][0] = bv[mb] ? ldg16(p) : uint4{0, 0, 0, 0};
          f.b[u][mb][BM == B_F32_SPLIT ? 1 : 0] = bv[mb] ? ldg16(p + 16) : uint4{0, 0, 0, 0};
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
  if (g.ks > 1 && !splitk_combine<NT, MT, LDT>(g, tile, tile_id, ksi, &s_flag)) return;

  const TileView v{tile, LDT, NT, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(g, e, v, s_epoch, Mtot, &s_flag);
}

// ------------------------------------------------------------------ fp32 VALU kernel
// fp32 configurations are small; one thread per (row, token) dot product, k
// ascending with fused multiply-adds.
template <int NT, int NMAT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(const GemmDesc g, const EpiDesc e) {
  constexpr int MT = 16, LDT = MT + 1, RPM = NT / NMAT;
  __shared__ float tile[NT * LDT];
  __shared__ int s_flag;
  __shared__ uint32_t s_epoch;
  const int tile_id = blockIdx.x / g.ks;
  const int m0 = blockIdx.y * MT;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;
  const int mcnt = min(MT, Mtot - m0);
  const int n0 = tile_id * RPM;
  if (EPI == EPI_TWELL && threadIdx.x == 0) s_epoch = atomic_load_agent(&g.ctrl[CTRL_EPOCH]) + 1u;
  for (int p = threadIdx.x; p < NT * mcnt; p += blockDim.x) {
    const int r = p % NT, m = p / NT;
    const int mat = r / RPM, rr = n0 + (r % RPM);
    const float* a = reinterpret_cast<const float*>(mat ? g.A1 : g.A0) + (size_t)rr * g.lda;
    const int row = g.gather ? g.gather[m0 + m] : m0 + m;
    const float* b = reinterpret_cast<const float*>(g.B) + (size_t)row * g.ldb;
    float s = 0.f;
    for (int k = 0; k < g.K; k += 4) {
      const float4 av = *reinterpret_cast<const float4*>(a + k);
      const float4 bw = *reinterpret_cast<const float4*>(b + k);
      s = fmaf(av.x, bw.x, s);
      s = fmaf(av.y, bw.y, s);
      s = fmaf(av.z, bw.z, s);
      s = fmaf(av.w, bw.w, s);
    }
    tile[r * LDT + m] = s;
  }
  __syncthreads();
  const TileView v{tile, LDT, NT, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(g, e, v, s_epoch, Mtot, &s_flag);
}

// ------------------------------------------------------------------ dispatch
template <int RB, int WN, int MB, int BM, int NMAT, int EPI>
static hipError_t go_bf16(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_bf16<RB, WN, MB, BM, NMAT, EPI>), grid, dim3(256), 0, s, g, e);
  return hipGetLastError();
}

template <int RB, int WN, int BM, int NMAT, int EPI>
static hipError_t pick_mb(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  switch (g.mt) {
    case 16: return go_bf16<RB, WN, 1, BM, NMAT, EPI>(g, e, grid, s);
    case 32: return go_bf16<RB, WN, 2, BM, NMAT, EPI>(g, e, grid, s);
    case 64: return go_bf16<RB, WN, 4, BM, NMAT, EPI>(g, e, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int BM, int NMAT, int EPI>
static hipError_t pick_nt(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  switch (g.nt) {
    case 16: if (NMAT == 1) return pick_mb<1, 1, BM, NMAT, EPI>(g, e, grid, s); break;
    case 32: return pick_mb<1, 2, BM, NMAT, EPI>(g, e, grid, s);
    case 64: return pick_mb<1, 4, BM, NMAT, EPI>(g, e, grid, s);
    case 128: return pick_mb<2, 4, BM, NMAT, EPI>(g, e, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int NMAT, int EPI>
static hipError_t go_f32(const GemmDesc& g, const EpiDesc& e, dim3 grid, hipStream_t s) {
  switch (g.nt) {
    case 16: if (NMAT == 1) { hipLaunchKernelGGL((k_gemm_f32<16, NMAT, EPI>), grid, dim3(256), 0, s, g, e); return hipGetLastError(); } break;
    case 32: hipLaunchKernelGGL((k_gemm_f32<32, NMAT, EPI>), grid, dim3(256), 0, s, g, e); return hipGetLastError();
    case 64: hipLaunchKernelGGL((k_gemm_f32<64, NMAT, EPI>), grid, dim3(256), 0, s, g, e); return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  const int tiles = g.nrows * g.nmat / g.nt;
  dim3 grid(tiles * g.ks, (g.M + g.mt - 1) / g.mt);
  if (g.dtype == DT_F32) {
    if (g.mt != 16 || g.ks != 1) return hipErrorInvalidValue;
    switch (e.kind) {
      case EPI_STORE_F32: return go_f32<1, EPI_STORE_F32>(g, e, grid, s);
      case EPI_TWELL: return go_f32<1, EPI_TWELL>(g, e, grid, s);
      case EPI_WINA: return go_f32<2, EPI_WINA>(g, e, grid, s);
      case EPI_DENSE_H: return g.nmat == 2 ? go_f32<2, EPI_DENSE_H>(g, e, grid, s) : go_f32<1, EPI_DENSE_H>(g, e, grid, s);
      case EPI_Y: return go_f32<1, EPI_Y>(g, e, grid, s);
    }
    return hipErrorInvalidValue;
  }
  const bool split = g.bmode == B_F32_SPLIT;
  switch (e.kind) {
    case EPI_STORE_F32:
      return split ? pick_nt<B_F32_SPLIT, 1, EPI_STORE_F32>(g, e, grid, s) : pick_nt<B_NATIVE, 1, EPI_STORE_F32>(g, e, grid, s);
    case EPI_TWELL:
      return split ? pick_nt<B_F32_SPLIT, 1, EPI_TWELL>(g, e, grid, s) : pick_nt<B_NATIVE, 1, EPI_TWELL>(g, e, grid, s);
    case EPI_WINA:
      return pick_nt<B_NATIVE, 2, EPI_WINA>(g, e, grid, s);
    case EPI_DENSE_H:
      return g.nmat == 2 ? pick_nt<B_NATIVE, 2, EPI_DENSE_H>(g, e, grid, s) : pick_nt<B_NATIVE, 1, EPI_DENSE_H>(g, e, grid, s);
    case EPI_Y:
      return pick_nt<B_NATIVE, 1, EPI_Y>(g, e, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ffn
