// Gated subspace inference for a linear map y = W x on gfx950 (bf16 weights
// and tokens, fp32 accumulation). Source: "Gated Subspace Inference for
// Transformer Acceleration", section 2.1 (x = V_k g + r, y = M g + W r with
// the cached image M = W V_k) and section 2.2 (per-token gate on
// rho = ||r|| / ||x||: below eps y = M g, otherwise y = W x).
//
// Decode-shaped: up to 16 tokens per launch group, every product a weight
// stream at about one FLOP per byte, so each kernel reads its matrix once,
// with all of a lane's loads in flight before the first is used:
//
//   k_gsi_proj   g = V_k^T x: rows of the transposed basis (k x d) cut into
//                up to 8 items of 512-element chunks, one item per wave; the
//                items of a row are added in order.
//   k_gsi_resid  ||x - V_k g||^2 and ||x||^2: rows of V_k (k elements,
//                lpr lanes of 8 each, several rows per wave instruction),
//                g staged in LDS; one part per row block and token (at most
//                64 row blocks at these shapes), a workgroup per row block
//                and chunk of up to 4 tokens.
//   k_gsi_out    the image rows (k elements, same lane layout) are loaded
//                first, since the fast path is the common case; then every
//                workgroup adds the parts in the same fixed order and takes
//                the same per-token gate (a kernel boundary orders the parts
//                before their readers, with no fence or ticket); fast tokens
//                get y = M g, slow tokens stream W's rows (one wave per row,
//                8 chunks of 16 bytes per lane in flight).
//
// With an orthonormal basis ||r||^2 = ||x||^2 - ||g||^2, but a bf16 basis is
// only nearly orthonormal and the difference cancels badly near the
// threshold, so the residual is formed explicitly (one more 2 MB stream at
// d = 4096, k = 256).
#include <algorithm>

#include "common.cuh"
#include "gsi.cuh"
#include "wave.cuh"

namespace ffn {

namespace {

// Sum of each v[i] over every aligned group of `lpr` lanes (a power of two,
// wave-uniform); every lane of a group ends with the group's total.
template <int V>
__device__ __forceinline__ void group_sum(float (&v)[V], int lpr) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (lpr > 32) v[i] += wave_xchg<32>(v[i]);
    if (lpr > 16) v[i] += wave_xchg<16>(v[i]);
    if (lpr > 8) v[i] += wave_xchg<8>(v[i]);
    if (lpr > 4) v[i] += wave_xchg<4>(v[i]);
    if (lpr > 2) v[i] += wave_xchg<2>(v[i]);
    if (lpr > 1) v[i] += wave_xchg<1>(v[i]);
  }
}

int pow2ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// k-rows a lane of the residual kernel holds: the fewest (1, 2, 4, 8) that
// keep its workgroups at most kGsiResParts, and at most kGsiResRowsMax rows
// per workgroup (rpi rows per wave instruction).
int res_nl_for(int d, int rpi) {
  const int vmax = std::min(kGsiMaxNl, kGsiResRowsMax / (kGsiResWaves * rpi));
  int v = 1;
  while (v < vmax && (d + kGsiResWaves * rpi * v - 1) / (kGsiResWaves * rpi * v) > kGsiResParts) v <<= 1;
  return v;
}

int group_maxm(int M) { return M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 8 : 16))); }

}  // namespace

// ------------------------------------------------------------------ g = V_k^T x
template <int MAXM>
__global__ __launch_bounds__(512) void k_gsi_proj(const GsiDesc d) {
  __shared__ float s_part[8 * MAXM];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int ipr = d.proj_ipr, npl = d.proj_npl;
  const int r = wave / ipr, s = wave - r * ipr;
  const int row = blockIdx.x * d.proj_rpb + r;
  const bool live = row < d.k;
  const uint16_t* vrow = d.vt + (size_t)(live ? row : 0) * d.d;
  uint4 a[kGsiProjMaxNpl];
#pragma unroll
  for (int i = 0; i < kGsiProjMaxNpl; ++i) {
    const int col = (s * npl + i) * 512 + lane * 8;
    a[i] = (live && i < npl && col < d.d) ? ldg16(vrow + col) : uint4{0, 0, 0, 0};
  }
  float acc[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) acc[m] = 0.f;
#pragma unroll
  for (int i = 0; i < kGsiProjMaxNpl; ++i) {
    const int col = (s * npl + i) * 512 + lane * 8;
    if (live && i < npl && col < d.d) {
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        if (m < d.M) acc[m] = dot8_bf(a[i], ldg16(d.x + (size_t)m * d.d + col), acc[m]);
    }
  }
  WaveTRed<MAXM, 32>::run(acc, lane);
  constexpr int SH = 6 - Log2<MAXM>::value;
  if ((lane & ((1 << SH) - 1)) == 0) s_part[wave * MAXM + (lane >> SH)] = acc[0];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < d.proj_rpb * MAXM) {
    const int rr = t / MAXM, m = t - rr * MAXM;
    const int rw = blockIdx.x * d.proj_rpb + rr;
    float g = 0.f;
    for (int q = 0; q < ipr; ++q) g += s_part[(rr * ipr + q) * MAXM + m];
    if (rw < d.k && m < d.M) d.g[(size_t)m * d.k + rw] = g;
  }
}

// ------------------------------------------------------------------ residual norms
// Workgroup (w, c) writes part[0][m][w] = sum over its rows j of
// (x_j - (V_k g)_j)^2 and part[1][m][w] = sum of x_j^2 for the tokens m of
// chunk c (TQ tokens: a bounded unroll, and more workgroups for more tokens;
// the chunks share the V_k rows through the cache).
template <int TQ>
__global__ __launch_bounds__(64 * kGsiResWaves) void k_gsi_resid(const GsiDesc d) {
  __shared__ float4 s_g4[TQ * kGsiMaxK / 4];          // g of the chunk's tokens [TQ x k]
  __shared__ float s_red[kGsiResWaves * 2 * TQ];
  __shared__ uint16_t s_x[TQ * kGsiResRowsMax];
  const float* s_g = reinterpret_cast<const float*>(s_g4);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int lpr = d.lpr, rpi = 64 / lpr, c8 = lane & (lpr - 1), rsub = lane / lpr;
  const int col = c8 * 8;
  const int rows_wg = kGsiResWaves * rpi * d.res_nl;
  const int j0 = blockIdx.x * rows_wg;
  const int m0 = blockIdx.y * TQ, mt = min(TQ, d.M - m0);
  uint4 a[kGsiMaxNl];
#pragma unroll
  for (int i = 0; i < kGsiMaxNl; ++i) {
    const int j = j0 + (i * kGsiResWaves + wave) * rpi + rsub;
    a[i] = (i < d.res_nl && j < d.d && col < d.k) ? ldg16(d.vk + (size_t)j * d.k + col) : uint4{0, 0, 0, 0};
  }
  // the chunk's x values on the workgroup's rows, and its g, staged once
  for (int p = threadIdx.x; p < mt * rows_wg; p += 64 * kGsiResWaves) {
    const int t = p / rows_wg, jj = p - t * rows_wg;
    s_x[p] = j0 + jj < d.d ? d.x[(size_t)(m0 + t) * d.d + j0 + jj] : (uint16_t)0;
  }
  const int n4 = mt * d.k / 4;
  for (int p = threadIdx.x; p < n4; p += 64 * kGsiResWaves)
    s_g4[p] = reinterpret_cast<const float4*>(d.g + (size_t)m0 * d.k)[p];
  __syncthreads();

  float rr[TQ], xx[TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t) rr[t] = xx[t] = 0.f;
#pragma unroll
  for (int i = 0; i < kGsiMaxNl; ++i) {
    if (i < d.res_nl) {
      const int j = j0 + (i * kGsiResWaves + wave) * rpi + rsub;
      float p[TQ];
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        p[t] = 0.f;
        if (t < mt && col < d.k) {
          const float4 b0 = *reinterpret_cast<const float4*>(s_g + t * d.k + col);
          const float4 b1 = *reinterpret_cast<const float4*>(s_g + t * d.k + col + 4);
          p[t] = dot8_f32(a[i], b0, b1, 0.f);
        }
      }
      group_sum(p, lpr);                          // (V_k g)_j in every lane of the row's group
      if (c8 == 0 && j < d.d) {
#pragma unroll
        for (int t = 0; t < TQ; ++t)
          if (t < mt) {
            const float xv = bf2f(s_x[t * rows_wg + (j - j0)]);
            const float rv = xv - p[t];
            rr[t] = fmaf(rv, rv, rr[t]);
            xx[t] = fmaf(xv, xv, xx[t]);
          }
      }
    }
  }
  float v[2 * TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    v[t] = rr[t];
    v[TQ + t] = xx[t];
  }
  WaveTRed<2 * TQ, 32>::run(v, lane);
  constexpr int SH = 6 - Log2<2 * TQ>::value;
  if ((lane & ((1 << SH) - 1)) == 0) s_red[wave * 2 * TQ + (lane >> SH)] = v[0];
  __syncthreads();
  if ((int)threadIdx.x < 2 * TQ) {
    const int q = threadIdx.x, which = q / TQ, t = q - which * TQ;
    float tot = 0.f;
    for (int w = 0; w < kGsiResWaves; ++w) tot += s_red[w * 2 * TQ + q];
    if (t < mt) d.part[((size_t)which * kGsiMaxM + m0 + t) * d.nres + blockIdx.x] = tot;
  }
}

// The per-token gate, taken the same way by every workgroup of the output
// kernel: the residual parts of every token (in LDS when they fit, else read
// in place), each token's sums in a fixed order (lane order within a chunk of
// 64 parts, chunks in order, the wave butterfly; one wave per token), then
// rho = sqrt(rr) / sqrt(xx) and fast <=> rho < eps. Workgroup 0 also writes
// rho, the slow-token list and its count. Returns the fast-token mask.
__device__ __forceinline__ uint32_t gsi_decide(const GsiDesc& d, float* s_parts, float* s_rho) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int half = d.M * d.nres;                   // parts of the group's tokens, per kind
  const bool in_lds = d.nres <= kGsiResParts;
  if (in_lds) {
    for (int q = threadIdx.x; q < 2 * half; q += blockDim.x) {
      const int which = q >= half ? 1 : 0, off = which * (kGsiMaxM * d.nres) + (q - which * half);
      s_parts[off] = d.part[off];
    }
    __syncthreads();
  }
  const float* src = in_lds ? s_parts : d.part;
  for (int m = wave; m < d.M; m += nw) {
    float ra = 0.f, xa = 0.f;
    for (int p0 = 0; p0 < d.nres; p0 += 64) {
      const int p = p0 + lane;
      if (p < d.nres) {
        ra += src[(size_t)m * d.nres + p];
        xa += src[((size_t)kGsiMaxM + m) * d.nres + p];
      }
    }
    ra = wave_sum(ra);
    xa = wave_sum(xa);
    if (lane == 0) s_rho[m] = xa > 0.f ? sqrtf(ra) / sqrtf(xa) : 0.f;     // x = 0: rho = 0
  }
  __syncthreads();
  uint32_t fast = 0;
  for (int m = 0; m < d.M; ++m)
    if (s_rho[m] < d.eps) fast |= 1u << m;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int n = d.tok0 > 0 ? *d.counter : 0;
    for (int m = 0; m < d.M; ++m) {
      if (d.rho) d.rho[d.tok0 + m] = s_rho[m];
      if (!((fast >> m) & 1u)) {
        if (d.slow_list) d.slow_list[n] = d.tok0 + m;
        ++n;
      }
    }
    *d.counter = n;
    if (d.n_slow) *d.n_slow = n;
  }
  return fast;
}

// Slow tokens of the output kernel: y = W x, one wave per W row (rows
// o0 + wave * rpw .. + rpw - 1): its chunks of 4096 inputs (8 x 16 bytes per
// lane in flight), each chunk's dot with every slow token, the chunk totals
// added in order into the wave's fp32 accumulators in LDS.
template <int TQ>
__device__ __forceinline__ void gsi_slow_rows(const GsiDesc& d, uint32_t slow, int o0, int rpw, float* yacc) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int P = (d.d + 511) / 512;
  constexpr int SH = 6 - Log2<TQ>::value;
  for (int q = 0; q < rpw; ++q) {
    const int o = o0 + wave * rpw + q;
    if (o >= d.dout) break;
    const uint16_t* wr = d.w + (size_t)o * d.d;
    if (lane < kGsiMaxM) yacc[lane] = 0.f;
    for (int c0 = 0; c0 < P; c0 += 8) {
      uint4 wv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int cc = (c0 + i) * 512 + lane * 8;
        wv[i] = cc < d.d ? ldg16(wr + cc) : uint4{0, 0, 0, 0};
      }
      for (int m0 = 0; m0 < d.M; m0 += TQ) {
        if (!((slow >> m0) & ((1u << TQ) - 1u))) continue;
        float acc[TQ];
#pragma unroll
        for (int t = 0; t < TQ; ++t) acc[t] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int cc = (c0 + i) * 512 + lane * 8;
          if (cc < d.d) {
#pragma unroll
            for (int t = 0; t < TQ; ++t)
              if ((slow >> (m0 + t)) & 1u)
                acc[t] = dot8_bf(wv[i], ldg16(d.x + (size_t)(m0 + t) * d.d + cc), acc[t]);
          }
        }
        WaveTRed<TQ, 32>::run(acc, lane);
        if ((lane & ((1 << SH) - 1)) == 0) {
          const int m = m0 + (lane >> SH);
          if (m < kGsiMaxM) yacc[m] += acc[0];
        }
      }
    }
    if (lane < d.M && ((slow >> lane) & 1u)) d.y[(size_t)lane * d.dout + o] = (uint16_t)f2bf(yacc[lane]);
  }
}

// ------------------------------------------------------------------ gate, then y = M g or W x
// Every workgroup takes the same decision from the residual parts (the same
// loads and sums in the same order); workgroup 0 also writes rho, the slow
// list and its count. Tokens are taken TQ at a time, as in the residual kernel.
// NC: 16-byte chunks of an image row per lane (1, or 4 with several tokens:
// fewer lanes per row, so each token's row sum takes fewer butterfly levels
// per multiply-add).
template <int TQ, int NC>
__global__ __launch_bounds__(256) void k_gsi_out(const GsiDesc d) {
  extern __shared__ float4 s_dyn4[];
  const float* s_g = reinterpret_cast<const float*>(s_dyn4);     // [M x k]
  __shared__ float s_parts[2 * kGsiMaxM * kGsiResParts];
  __shared__ float s_rho[kGsiMaxM];
  __shared__ float s_yacc[4][kGsiMaxM];
  constexpr int NLMAX = NC == 1 ? kGsiMaxNl : 2;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int lpr = NC == 1 ? d.lpr : d.lpr4, rpi = 64 / lpr, c8 = lane & (lpr - 1), rsub = lane / lpr;
  const int nl = NC == 1 ? d.out_nl : d.out_nl4;
  const int col = c8 * 8;             // chunk c of a lane: elements (c * lpr + c8) * 8 ...
  const int rows_wg = 4 * rpi * nl;
  const int o0 = blockIdx.x * rows_wg;
  // image rows first: they are needed unless every token is slow
  uint4 a[NLMAX][NC];
#pragma unroll
  for (int i = 0; i < NLMAX; ++i) {
    const int o = o0 + (i * 4 + wave) * rpi + rsub;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int cc = col + c * lpr * 8;
      a[i][c] = (!d.force_slow && i < nl && o < d.dout && cc < d.k) ? ldg16(d.img + (size_t)o * d.k + cc)
                                                                     : uint4{0, 0, 0, 0};
    }
  }
  const uint32_t all = (1u << d.M) - 1u;
  const uint32_t fast = d.force_slow ? 0u : gsi_decide(d, s_parts, s_rho);
  const uint32_t slow = all & ~fast;

  if (fast) {
    const int n4 = d.M * d.k / 4;
    for (int p = threadIdx.x; p < n4; p += 256) s_dyn4[p] = reinterpret_cast<const float4*>(d.g)[p];
    __syncthreads();
    for (int m0 = 0; m0 < d.M; m0 += TQ) {
      if (!((fast >> m0) & ((1u << TQ) - 1u))) continue;
#pragma unroll
      for (int i = 0; i < NLMAX; ++i) {
        if (i < nl) {
          const int o = o0 + (i * 4 + wave) * rpi + rsub;
          float p[TQ];
#pragma unroll
          for (int t = 0; t < TQ; ++t) {
            const int m = m0 + t;
            p[t] = 0.f;
            if ((fast >> m) & 1u) {
#pragma unroll
              for (int c = 0; c < NC; ++c) {
                const int cc = col + c * lpr * 8;
                if (cc < d.k) {
                  const float4 b0 = *reinterpret_cast<const float4*>(s_g + m * d.k + cc);
                  const float4 b1 = *reinterpret_cast<const float4*>(s_g + m * d.k + cc + 4);
                  p[t] = dot8_f32(a[i][c], b0, b1, p[t]);
                }
              }
            }
          }
          group_sum(p, lpr);
          if (c8 == 0 && o < d.dout) {
#pragma unroll
            for (int t = 0; t < TQ; ++t)
              if ((fast >> (m0 + t)) & 1u) d.y[(size_t)(m0 + t) * d.dout + o] = (uint16_t)f2bf(p[t]);
          }
        }
      }
    }
  }

  if (slow) gsi_slow_rows<TQ>(d, slow, o0, rows_wg / 4, s_yacc[wave]);
}

// The output kernel with 8..16 tokens on matrix cores: wave w owns 16 image
// rows, one 16 x 16 tile of y over the tokens, y[o][m] = sum_c M[o][c] g[m][c]
// as v_mfma_f32_16x16x32_bf16 steps over c with g split into bf16 hi + lo (two
// products a step; the products are exact and summed in fp32). Operand lane
// l holds image row l % 16 (A) or token l % 16 (B), elements 8 (l / 16) .. +7
// of the step's 32; the image rows and g are loaded before the gate is taken.
// g sits in LDS with rows padded by 4 floats, so the 16 tokens of a read fall
// in distinct banks. Slow tokens take the same path as in k_gsi_out.
__global__ __launch_bounds__(256) void k_gsi_out_mf(const GsiDesc d) {
  extern __shared__ float4 s_dyn4[];
  float* s_g = reinterpret_cast<float*>(s_dyn4);                 // [M x (k + 4)]
  __shared__ float s_parts[2 * kGsiMaxM * kGsiResParts];
  __shared__ float s_rho[kGsiMaxM];
  __shared__ float s_yacc[4][kGsiMaxM];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int o0 = blockIdx.x * 64, ob = o0 + wave * 16;
  const int steps = d.k / 32, ldg = d.k + 4;
  uint4 aw[kGsiMaxK / 32];
  {
    const int orow = ob + r16;
#pragma unroll
    for (int j = 0; j < kGsiMaxK / 32; ++j)
      aw[j] = (!d.force_slow && j < steps && orow < d.dout) ? ldg16(d.img + (size_t)orow * d.k + 32 * j + 8 * q)
                                                             : uint4{0, 0, 0, 0};
  }
  // g of the group too, in the same round as the image rows (it does not
  // depend on the gate): at most 16 x 512 floats, 8 float4 a thread
  const int k4 = d.k / 4, n4 = d.M * k4;
  float4 gq[kGsiMaxM * kGsiMaxK / 4 / 256];
#pragma unroll
  for (int u = 0; u < kGsiMaxM * kGsiMaxK / 4 / 256; ++u) {
    const int p = threadIdx.x + 256 * u;
    gq[u] = (!d.force_slow && p < n4) ? reinterpret_cast<const float4*>(d.g)[p] : float4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t all = (1u << d.M) - 1u;
  const uint32_t fast = d.force_slow ? 0u : gsi_decide(d, s_parts, s_rho);
  const uint32_t slow = all & ~fast;

  if (fast) {
#pragma unroll
    for (int u = 0; u < kGsiMaxM * kGsiMaxK / 4 / 256; ++u) {
      const int p = threadIdx.x + 256 * u, m = p / k4, c = p - m * k4;
      if (p < n4) *reinterpret_cast<float4*>(s_g + (size_t)m * ldg + 4 * c) = gq[u];
    }
    __syncthreads();
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float* gr = s_g + (size_t)min(r16, d.M - 1) * ldg + 8 * q;
#pragma unroll
    for (int j = 0; j < kGsiMaxK / 32; ++j) {
      if (j < steps) {
        const float4 g0 = *reinterpret_cast<const float4*>(gr + 32 * j);
        const float4 g1 = *reinterpret_cast<const float4*>(gr + 32 * j + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = r16 < d.M ? gv[e] : 0.f;
          hi[e] = f2bf(v);
          lo[e] = f2bf(v - bf2f(hi[e]));
        }
        const uint4 bh{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
        const uint4 bl{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw[j]), as_bf16x8(bh), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw[j]), as_bf16x8(bl), acc, 0, 0, 0);
      }
    }
    // lane l: rows ob + 4 (l / 16) + v, token l % 16
    if (r16 < d.M && ((fast >> r16) & 1u)) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = ob + 4 * q + v;
        if (o < d.dout) d.y[(size_t)r16 * d.dout + o] = (uint16_t)f2bf(acc[v]);
      }
    }
  }
  if (slow) gsi_slow_rows<4>(d, slow, o0, 16, s_yacc[wave]);
}

// ------------------------------------------------------------------ image M = W V_k (set-up)
__global__ __launch_bounds__(256) void k_gsi_image(const uint16_t* __restrict__ w, const uint16_t* __restrict__ vt,
                                                  uint16_t* __restrict__ img, int dout, int d, int k) {
  __shared__ float sw[32][65];      // [j][o]
  __shared__ float sv[32][65];      // [j][c]
  const int o0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int lr = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 8;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int l = 0; l < 4; ++l) acc[i][l] = 0.f;
  for (int j0 = 0; j0 < d; j0 += 32) {
    const int jj = j0 + lc;
    const uint4 wv = (o0 + lr < dout && jj < d) ? ldg16(w + (size_t)(o0 + lr) * d + jj) : uint4{0, 0, 0, 0};
    const uint4 vv = (c0 + lr < k && jj < d) ? ldg16(vt + (size_t)(c0 + lr) * d + jj) : uint4{0, 0, 0, 0};
    float fw[8], fv[8];
    unpack8(wv, fw);
    unpack8(vv, fv);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sw[lc + e][lr] = fw[e];
      sv[lc + e][lr] = fv[e];
    }
    __syncthreads();
    for (int jx = 0; jx < 32; ++jx) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = sw[jx][ty * 4 + i];
        bv[i] = sv[jx][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int l = 0; l < 4; ++l) acc[i][l] = fmaf(av[i], bv[l], acc[i][l]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int o = o0 + ty * 4 + i, c = c0 + tx * 4 + l;
      if (o < dout && c < k) img[(size_t)o * k + c] = (uint16_t)f2bf(acc[i][l]);
    }
}

// ------------------------------------------------------------------ plans and launches
bool gsi_plan(GsiDesc& d, int cus) {
  if (d.d < 8 || d.d % 8 != 0 || d.d > 16384 || d.k < 8 || d.k % 8 != 0 || d.k > 512 || d.k > d.d || d.dout < 1)
    return false;
  const int P = (d.d + 511) / 512;
  d.proj_ipr = std::min(8, pow2ceil(P));
  d.proj_npl = (P + d.proj_ipr - 1) / d.proj_ipr;
  d.proj_rpb = 8 / d.proj_ipr;
  if (d.proj_npl > kGsiProjMaxNpl) return false;
  d.lpr = pow2ceil(d.k / 8);
  const int rpi = 64 / d.lpr;
  // residual: the fewest rows a lane holds that keeps the parts at most
  // kGsiResParts (every output workgroup reads them all); output: the most
  // rows a lane holds that still gives two workgroups per CU
  d.res_nl = res_nl_for(d.d, rpi);
  d.nres = (d.d + kGsiResWaves * rpi * d.res_nl - 1) / (kGsiResWaves * rpi * d.res_nl);
  d.out_nl = 1;
  for (int v = kGsiMaxNl; v >= 1; v >>= 1) {
    if ((d.dout + 4 * rpi * v - 1) / (4 * rpi * v) >= 2 * cus) {
      d.out_nl = v;
      break;
    }
  }
  d.nout = (d.dout + 4 * rpi * d.out_nl - 1) / (4 * rpi * d.out_nl);
  // several tokens: 4 chunks (32 elements) of an image row per lane
  d.lpr4 = pow2ceil((d.k + 31) / 32);
  const int rpi4 = 64 / d.lpr4;
  d.out_nl4 = (d.dout + 4 * rpi4 * 2 - 1) / (4 * rpi4 * 2) >= 2 * cus ? 2 : 1;
  d.nout4 = (d.dout + 4 * rpi4 * d.out_nl4 - 1) / (4 * rpi4 * d.out_nl4);
  return true;
}

// Largest number of residual workgroups any plan gives for this shape (the
// workspace holds that many parts).
int gsi_max_parts(int d_in, int k) {
  const int rpi = 64 / pow2ceil(k / 8);
  const int rows = kGsiResWaves * rpi * res_nl_for(d_in, rpi);
  return (d_in + rows - 1) / rows;
}

hipError_t launch_gsi_proj(const GsiDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kGsiMaxM || d.proj_rpb * d.proj_ipr != 8) return hipErrorInvalidValue;
  const dim3 grid((d.k + d.proj_rpb - 1) / d.proj_rpb), blk(512);
  switch (group_maxm(d.M)) {
    case 1: ffn_launch(k_gsi_proj<1>, grid, blk, 0, s, d); break;
    case 2: ffn_launch(k_gsi_proj<2>, grid, blk, 0, s, d); break;
    case 4: ffn_launch(k_gsi_proj<4>, grid, blk, 0, s, d); break;
    case 8: ffn_launch(k_gsi_proj<8>, grid, blk, 0, s, d); break;
    default: ffn_launch(k_gsi_proj<16>, grid, blk, 0, s, d); break;
  }
  return hipGetLastError();
}

hipError_t launch_gsi_resid(const GsiDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kGsiMaxM || d.res_nl < 1 || d.res_nl > kGsiMaxNl || d.nres < 1) return hipErrorInvalidValue;
  const int tq = std::min(group_maxm(d.M), 4);
  const dim3 grid(d.nres, (d.M + tq - 1) / tq), blk(64 * kGsiResWaves);
  switch (tq) {
    case 1: ffn_launch(k_gsi_resid<1>, grid, blk, 0, s, d); break;
    case 2: ffn_launch(k_gsi_resid<2>, grid, blk, 0, s, d); break;
    default: ffn_launch(k_gsi_resid<4>, grid, blk, 0, s, d); break;
  }
  return hipGetLastError();
}

hipError_t launch_gsi_out(const GsiDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kGsiMaxM || d.out_nl < 1 || d.out_nl > kGsiMaxNl || d.nout < 1 || d.out_nl4 < 1 ||
      d.out_nl4 > 2 || d.nout4 < 1)
    return hipErrorInvalidValue;
  const dim3 blk(256);
  if (group_maxm(d.M) >= 8 && d.k % 32 == 0) {
    // 8..16 tokens: the matrix-core output kernel, 64 image rows a workgroup
    ffn_launch(k_gsi_out_mf, dim3((d.dout + 63) / 64), blk, (size_t)d.M * (d.k + 4) * 4, s, d);
    return hipGetLastError();
  }
  const size_t lds = (size_t)d.M * d.k * 4;
  switch (std::min(group_maxm(d.M), 4)) {
    case 1: ffn_launch((k_gsi_out<1, 1>), dim3(d.nout), blk, lds, s, d); break;
    case 2: ffn_launch((k_gsi_out<2, 1>), dim3(d.nout), blk, lds, s, d); break;
    default: ffn_launch((k_gsi_out<4, 4>), dim3(d.nout4), blk, lds, s, d); break;
  }
  return hipGetLastError();
}

hipError_t launch_gsi_image(const uint16_t* w, const uint16_t* vt, uint16_t* img, int dout, int d, int k,
                            hipStream_t s) {
  if (dout < 1 || d < 8 || d % 8 != 0 || k < 1) return hipErrorInvalidValue;
  const dim3 grid((dout + 63) / 64, (k + 63) / 64);
  ffn_launch(k_gsi_image, grid, dim3(256), 0, s, w, vt, img, dout, d, k);
  return hipGetLastError();
}

}  // namespace ffn
