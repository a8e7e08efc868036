// Decode path of the sparse gated FFN on gfx950: bf16 weights, 1..16 tokens,
// ReLU gate with a bias or threshold selection.
//
// At a handful of tokens every product is a memory-bound weight stream
// (about one FLOP per byte), so the path is organised around reading each
// touched weight byte once, with all 256 CUs busy and every load of a wave
// issued before the first is used:
//
//   k_dec_lowrank  t = V x (low-rank gate only; LoPA page, "How LoPA Gating
//                  Restructures FFN Computation"): 1 KB pieces of V's rows,
//                  several per wave, reduced in LDS; from two tokens
//                  k_dec_lowrank_mf, the same product on matrix cores, as
//                  fp32 slabs over slices of d.
//   k_dec_gate     one workgroup per sub-tile of R gate rows (R divides the
//                  TwELL tile width T). The gate rows are streamed and dotted
//                  with every token (VALU, or matrix cores from 5 tokens with a
//                  low-rank gate and from 9 with a full one); the epilogue
//                  applies the selection and writes the TwELL pack straight
//                  from LDS (Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷"):
//                  a sub-tile learns its slot offset inside the TwELL tile from
//                  the counts the earlier sub-tiles publish (epoch-tagged
//                  words). Before it waits for those, the workgroup starts on
//                  the neurons active for any token (the sub-tile's union mask,
//                  one 64-bit word), in one of three organisations:
//     partial rows (one token): it reads the up and down rows of its active
//                  neurons in one memory round and writes one partial y row;
//                  k_dec_reduce adds the non-empty rows in sub-tile order.
//     chunk:       it stores h = a * <W_up[i,:], x> densely; k_dec_down (one
//                  workgroup per 16-byte column chunk of y) reads the union
//                  masks, deals their set bits to its threads and accumulates
//                  h * W_down^T[i, chunk] for every token.
//     split (2..16 tokens): it publishes the activations only; k_dec_up deals
//                  the union list evenly over 256 workgroups and runs the up
//                  products on matrix cores (bf16 h per list entry), and
//                  k_dec_down2 + k_dec_reduce2 run the down products on matrix
//                  cores over 64-column slices of y and entry groups.
//                  A token whose tile overflows the ELL width still has every
//                  active neuron in the lists, so no dense backup is needed at
//                  these token counts (Sparser/Faster/Lighter page, "Hybrid
//                  應對非均勻稀疏", routes busy rows; here they cost one more
//                  list entry per neuron). Every y element is summed in a fixed
//                  order, so y is bitwise reproducible; the last kernel's extra
//                  workgroup routes the pack.
#include <algorithm>
#include <type_traits>

#include "common.cuh"
#include "kernels.cuh"
#include "route.cuh"
#include "wave.cuh"

namespace ffn {

// ------------------------------------------------------------------ shared GEMV
// Dot products of rows [row0, row0 + R) of A (nrows x K bf16, row-major) with
// the MAXM token rows held in LDS (s_bf: bf16 [MAXM x K]; s_bf32: fp32
// [MAXM x K]). A row is P pieces of 512 elements (the last may be partly or
// wholly past K); the workgroup's R * P = NW * IPW pieces are dealt to the
// waves in row-major order, IPW consecutive pieces per wave.
// dec_gemv_issue starts the loads of a wave's pieces (they stay in flight
// while the caller stages the token inputs); dec_gemv_finish multiplies each
// piece's 8 elements per lane, reduces across the wave with WaveTRed and adds
// the piece sums of a row in piece order. Result: s_g[r * MAXM + m].
template <int NW, int IPW>
__device__ __forceinline__ void dec_gemv_issue(const uint16_t* __restrict__ A, int nrows, int K, int P, int row0,
                                               uint4 (&a)[IPW]) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = wave * IPW + i, r = q / P, c = q - r * P;
    const int col = c * 512 + lane * 8;
    const int row = row0 + r;
    a[i] = (col < K && row < nrows) ? ldg16(A + (size_t)row * K + col) : uint4{0, 0, 0, 0};
  }
}

template <int NW, int IPW, int MAXM, bool BF32>
__device__ __forceinline__ void dec_gemv_finish(const uint4 (&a)[IPW], int K, int P, const uint16_t* s_bf,
                                                const float* s_bf32, float* s_part, float* s_g) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int R = NW * IPW / P;
  constexpr int V = IPW * MAXM;
  float v[V];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int q = wave * IPW + i, c = q % P;
    const int col = c * 512 + lane * 8;
    const bool ok = col < K;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      float s = 0.f;
      if (ok) {
        if (BF32) {
          const float4 b0 = *reinterpret_cast<const float4*>(s_bf32 + (size_t)m * K + col);
          const float4 b1 = *reinterpret_cast<const float4*>(s_bf32 + (size_t)m * K + col + 4);
          s = dot8_f32(a[i], b0, b1, 0.f);
        } else {
          s = dot8_bf(a[i], *reinterpret_cast<const uint4*>(s_bf + (size_t)m * K + col), 0.f);
        }
      }
      v[i * MAXM + m] = s;
    }
  }
  WaveTRed<V, 32>::run(v, lane);
  constexpr int SH = 6 - Log2<V>::value;
  if (P == 1) {
    // one piece per row: the wave totals are the row values
    if ((lane & ((1 << SH) - 1)) == 0) {
      const int j = lane >> SH, i = j / MAXM, m = j % MAXM;
      s_g[(wave * IPW + i) * MAXM + m] = v[0];
    }
    __syncthreads();
    return;
  }
  if ((lane & ((1 << SH) - 1)) == 0) {
    const int j = lane >> SH, i = j / MAXM, m = j % MAXM;
    s_part[(wave * IPW + i) * MAXM + m] = v[0];
  }
  __syncthreads();
  for (int p = threadIdx.x; p < R * MAXM; p += NW * 64) {
    const int r = p / MAXM, m = p % MAXM;
    float g = 0.f;
    for (int c = 0; c < P; ++c) g += s_part[(r * P + c) * MAXM + m];
    s_g[r * MAXM + m] = g;
  }
  __syncthreads();
}

// Low-rank gate of 5..16 tokens on matrix cores: G[r, m] = U[n0 + r, :] t_m
// for the R = 16 * NG rows of a sub-tile. t is fp32 and is not rounded: it is
// split into bf16 hi + lo parts (t - hi rounded again), so each step is two
// exact-product v_mfma_f32_16x16x32_bf16 accumulating in fp32. Waves
// [g NW / NG, (g + 1) NW / NG) own row group g, each a contiguous range of
// DS = K / 32 / (NW / NG) steps; operand lane l holds row l % 16 (A) or token
// l % 16 (B, zero from M on) at the 16-byte chunk 4 j + l / 16.
template <int NW, int NG, int DS>
__device__ __forceinline__ void dec_mfma_issue(const uint16_t* __restrict__ A, int K, int row0, uint4 (&a)[DS]) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  constexpr int WPG = NW / NG;
  const int g = wave / WPG, j0 = (wave % WPG) * DS;
  const uint16_t* ar = A + (size_t)(row0 + g * 16 + (lane & 15)) * K + (lane >> 4) * 8;
#pragma unroll
  for (int j = 0; j < DS; ++j) a[j] = ldg16(ar + (j0 + j) * 32);
}

template <int NW, int NG, int DS, int MAXM>
__device__ __forceinline__ void dec_mfma_finish(const uint4 (&a)[DS], int K, const float* s_t, int M,
                                                f32x4_t* s_acc, float* s_g) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  constexpr int WPG = NW / NG;
  const int g = wave / WPG, j0 = (wave % WPG) * DS;
  const int q = lane >> 4, r16 = lane & 15;
  const float* tr = s_t + (size_t)min(r16, M - 1) * K + q * 8;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < DS; ++j) {
    const float4 t0 = *reinterpret_cast<const float4*>(tr + (j0 + j) * 32);
    const float4 t1 = *reinterpret_cast<const float4*>(tr + (j0 + j) * 32 + 4);
    const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h0 = r16 < M ? f2bf(tv[2 * e]) : 0u, h1 = r16 < M ? f2bf(tv[2 * e + 1]) : 0u;
      const uint32_t l0 = r16 < M ? f2bf(tv[2 * e] - bf2f(h0)) : 0u;
      const uint32_t l1 = r16 < M ? f2bf(tv[2 * e + 1] - bf2f(h1)) : 0u;
      hi[e] = h0 | (h1 << 16);
      lo[e] = l0 | (l1 << 16);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[j]), as_bf16x8(uint4{hi[0], hi[1], hi[2], hi[3]}), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[j]), as_bf16x8(uint4{lo[0], lo[1], lo[2], lo[3]}), acc, 0, 0, 0);
  }
  s_acc[wave * 64 + lane] = acc;
  __syncthreads();
  // row group g's WPG tiles summed in wave order; lane l of the group's first
  // wave holds rows 4 (l / 16) + v, token l % 16
  if (wave % WPG == 0) {
    f32x4_t s = s_acc[wave * 64 + lane];
#pragma unroll
    for (int w = 1; w < WPG; ++w) {
      const f32x4_t u = s_acc[(wave + w) * 64 + lane];
      s[0] += u[0];
      s[1] += u[1];
      s[2] += u[2];
      s[3] += u[3];
    }
    if (r16 < MAXM) {
#pragma unroll
      for (int v = 0; v < 4; ++v) s_g[(g * 16 + 4 * q + v) * MAXM + r16] = r16 < M ? s[v] : 0.f;
    }
  }
  __syncthreads();
}

// Full gate of 9..16 tokens on matrix cores: G[r, m] = W_gate[n0 + r, :] x_m for
// the 32 rows of a sub-tile (two 16-row groups of four waves). x is bf16, so
// one exact-product v_mfma_f32_16x16x32_bf16 per step; a wave owns ds = K / 128
// consecutive steps (at most 16), operand lane l holding row l % 16 (A) or
// token l % 16 (B, from LDS, zero from M on) at the 16-byte chunk 4 j + l / 16.
constexpr int kFgMaxSteps = 16;

__device__ __forceinline__ void dec_fg_issue(const uint16_t* __restrict__ A, int K, int row0,
                                             uint4 (&a)[kFgMaxSteps]) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int ds = K / 128, g = wave >> 2, j0 = (wave & 3) * ds;
  const uint16_t* ar = A + (size_t)(row0 + g * 16 + (lane & 15)) * K + (lane >> 4) * 8;
#pragma unroll
  for (int j = 0; j < kFgMaxSteps; ++j) a[j] = j < ds ? ldg16(ar + (j0 + j) * 32) : uint4{0, 0, 0, 0};
}

template <int MAXM>
__device__ __forceinline__ void dec_fg_finish(const uint4 (&a)[kFgMaxSteps], int K, const uint16_t* s_x, int M,
                                              f32x4_t* s_acc, float* s_g) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int ds = K / 128, g = wave >> 2, j0 = (wave & 3) * ds;
  const int q = lane >> 4, r16 = lane & 15;
  const uint16_t* xr = s_x + (size_t)min(r16, M - 1) * K + q * 8;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kFgMaxSteps; ++j) {
    if (j < ds) {
      uint4 b = *reinterpret_cast<const uint4*>(xr + (j0 + j) * 32);
      if (r16 >= M) b = uint4{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[j]), as_bf16x8(b), acc, 0, 0, 0);
    }
  }
  s_acc[wave * 64 + lane] = acc;
  __syncthreads();
  // group g's four tiles summed in wave order; lane l of the group's first
  // wave holds rows 4 (l / 16) + v, token l % 16
  if ((wave & 3) == 0) {
    f32x4_t t = s_acc[wave * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4_t u = s_acc[(wave + w) * 64 + lane];
      t[0] += u[0];
      t[1] += u[1];
      t[2] += u[2];
      t[3] += u[3];
    }
    if (r16 < MAXM) {
#pragma unroll
      for (int v = 0; v < 4; ++v) s_g[(g * 16 + 4 * q + v) * MAXM + r16] = r16 < M ? t[v] : 0.f;
    }
  }
  __syncthreads();
}

// Stages `rows` rows of `cols16` 16-byte chunks (row stride ld16 chunks in
// global memory) into LDS, zero-filling rows [rows, MAXM); up to 8 loads per
// thread in flight.
template <int MAXM>
__device__ __forceinline__ void stage_rows(uint4* dst, const uint4* src, int rows, int cols16, size_t ld16) {
  constexpr int NB = MAXM < 8 ? 2 * MAXM : 8;
  stage_lds<NB>(dst, MAXM * cols16, [&](int p) {
    const int m = p / cols16, c = p - m * cols16;
    return m < rows ? src[(size_t)m * ld16 + c] : uint4{0, 0, 0, 0};
  });
}

// ------------------------------------------------------------------ k_dec_lowrank
template <int IPW, int MAXM>
__device__ __forceinline__ void dec_lowrank_body(const DecodeDesc& d) {
  extern __shared__ uint4 s_dyn[];
  __shared__ float s_part[kDecVWaves * IPW * MAXM];
  __shared__ float s_g[kDecVWaves * IPW * MAXM];
  uint16_t* s_x = reinterpret_cast<uint16_t*>(s_dyn);
  const int P = d.ipw;                     // pieces per V row (power of two)
  const int R = kDecVWaves * IPW / P;
  const int row0 = blockIdx.x * R;
  uint4 a[IPW];
  dec_gemv_issue<kDecVWaves, IPW>(reinterpret_cast<const uint16_t*>(d.v), d.rank, d.d, P, row0, a);
  stage_rows<MAXM>(s_dyn, reinterpret_cast<const uint4*>(d.x), d.M, d.d / 8, d.d / 8);
  __syncthreads();
  dec_gemv_finish<kDecVWaves, IPW, MAXM, false>(a, d.d, P, s_x, nullptr, s_part, s_g);
  for (int p = threadIdx.x; p < R * MAXM; p += blockDim.x) {
    const int r = p / MAXM, m = p % MAXM;
    if (m < d.M && row0 + r < d.rank) d.t[(size_t)m * d.rank + row0 + r] = s_g[r * MAXM + m];
  }
}
template <int IPW, int MAXM>
__global__ __launch_bounds__(64 * kDecVWaves) void k_dec_lowrank(const DecodeDesc d) { dec_lowrank_body<IPW, MAXM>(d); }
template <int IPW, int MAXM>
__global__ __launch_bounds__(64 * kDecVWaves) void k_dec_lowrank_grp(const DecGroup g) { dec_lowrank_body<IPW, MAXM>(g.d[blockIdx.y]); }

// ------------------------------------------------------------------ k_dec_lowrank_mf
// t = V x for 2..16 tokens on matrix cores (bf16 inputs, exact products): a
// small dense contraction, 16 rows of V x d x the tokens per row group. The
// grid is (rank / 16 row groups) x (nslab slices of d); the NWV waves of a
// workgroup (blockDim / 64: 4, 8 or 16) split its slice, step j of a wave
// being one v_mfma_f32_16x16x32_bf16 with operand lane l holding row l % 16
// (A: V, B: token l % 16, zero from M on) at the 16-byte chunk 4 j + l / 16.
// The partial tiles are summed in LDS in wave order and written as slab z,
// fp32 [M x rank]; the gate kernel adds the nslab slabs in slab order. Few
// slabs keep the gate's reads of t small (every gate workgroup reads all of
// them); wide workgroups keep the first stage's loads in flight.
constexpr int kLrMaxWaves = 16;
constexpr int kLrMaxSteps = 8;                        // 32-element steps per wave

__device__ __forceinline__ void dec_lowrank_mf_body(const DecodeDesc& d) {
  __shared__ f32x4_t s_acc[kLrMaxWaves][64];
  const int lane = lane_id(), wave = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  const int q = lane >> 4, r16 = lane & 15, M = d.M, dm = d.d, z = blockIdx.y;
  const int steps = dm / (32 * nwv * d.nslab);
  const int k0 = (z * nwv + wave) * steps * 32;
  const int row = blockIdx.x * 16 + r16;
  const uint16_t* vr = reinterpret_cast<const uint16_t*>(d.v) + (size_t)row * dm + k0 + q * 8;
  const uint16_t* xr = reinterpret_cast<const uint16_t*>(d.x) + (size_t)min(r16, M - 1) * dm + k0 + q * 8;
  uint4 a[kLrMaxSteps], b[kLrMaxSteps];
#pragma unroll
  for (int j = 0; j < kLrMaxSteps; ++j) {
    a[j] = uint4{0, 0, 0, 0};
    b[j] = uint4{0, 0, 0, 0};
    if (j < steps) {                                   // uniform; B rows clamped, then masked
      a[j] = ldg16(vr + j * 32);
      const uint4 xv = ldg16(xr + j * 32);
      b[j] = r16 < M ? xv : uint4{0, 0, 0, 0};
    }
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kLrMaxSteps; ++j)
    if (j < steps) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[j]), as_bf16x8(b[j]), acc, 0, 0, 0);
  s_acc[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t t = s_acc[0][lane];
    for (int w = 1; w < nwv; ++w) {
      const f32x4_t u = s_acc[w][lane];
      t[0] += u[0];
      t[1] += u[1];
      t[2] += u[2];
      t[3] += u[3];
    }
    // lane l: rows 16 b + 4 (l / 16) + v, token l % 16
    if (r16 < M)
      *reinterpret_cast<float4*>(d.tslab + ((size_t)z * M + r16) * d.rank + blockIdx.x * 16 + 4 * q) =
          float4{t[0], t[1], t[2], t[3]};
  }
}
__global__ __launch_bounds__(64 * kLrMaxWaves) void k_dec_lowrank_mf(const DecodeDesc d) { dec_lowrank_mf_body(d); }
__global__ __launch_bounds__(64 * kLrMaxWaves) void k_dec_lowrank_mf_grp(const DecGroup g) { dec_lowrank_mf_body(g.d[blockIdx.z]); }

// Waves per workgroup of the matrix-core first stage for S slices of d (0: no
// shape fits): the fewest of 4, 8, 16 whose wave slices take at most
// kLrMaxSteps steps.
static int lowrank_mf_waves(int d_model, int S) {
  for (int nwv = 4; nwv <= kLrMaxWaves; nwv *= 2) {
    const int per = 32 * nwv * S;
    if (d_model % per == 0 && d_model / per <= kLrMaxSteps) return nwv;
  }
  return 0;
}

// Slices of d for the matrix-core first stage (0: not applicable, or the VALU
// kernel). `want` (a power of two, 0 for the default, negative for the VALU
// kernel up to 8 tokens) asks for a slice count.
int dec_lowrank_slabs(int m, int d_model, int rank, int want) {
  if (m < 2 || m > kDecMaxM || rank % 16 != 0 || d_model % 512 != 0) return 0;
  if (want < 0 && m <= 8) return 0;                    // the VALU first stage (t in one piece)
  int S = want > 0 ? want : 8;                       // 2, 4 or 8 slabs measure within 1 us at 2..8 tokens
  S = std::max(1, std::min(S, 8));
  while (S < 8 && lowrank_mf_waves(d_model, S) == 0) S *= 2;
  return lowrank_mf_waves(d_model, S) ? S : 0;
}

// ------------------------------------------------------------------ k_dec_gate
__device__ __forceinline__ float dec_bias(const DecodeDesc& d, int t) { return d.bias ? d.bias[t] : d.bias_scalar; }
__device__ __forceinline__ float dec_cut(const DecodeDesc& d, int t) {
  return d.sel == SEL_THRESH ? fmaxf(d.tau[t], 0.f) : 0.f;
}

// Waits (bounded) until an epoch-tagged look-back word carries this pass's
// epoch and returns its count.
__device__ __forceinline__ int lb_count(const uint64_t* p, const WaitCtl& wc, uint64_t first, uint32_t* ctrl) {
  return (int)tagged_wait(p, first, wc, ctrl);
}

template <int NW, int IPW, int MAXM, bool LOWRANK, int MODE>
__device__ __forceinline__ void dec_gate_body(const DecodeDesc& d) {
  constexpr bool PART = MODE == DEC_PART;
  extern __shared__ uint4 s_dyn[];
  __shared__ float s_part[NW * IPW * MAXM];
  __shared__ float s_g[64 * MAXM];
  __shared__ uint64_t s_bal[MAXM];
  __shared__ int s_urow[64];
  __shared__ float s_h[PART ? 64 * MAXM : 1];
  __shared__ f32x4_t s_acc[((LOWRANK && MAXM >= 8) || MAXM == 16) && NW == 8 ? NW * 64 : 1];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int M = d.M, dm = d.d, F = d.F;
  const int K = d.K;
  int P = 1;
  while (P * 512 < K) P <<= 1;
  // 9..16 tokens with a full gate: 32-row sub-tiles on matrix cores (the host
  // plans this shape only when K allows it)
  constexpr bool FG = !LOWRANK && MAXM == 16 && NW == 8;
  const int R = FG ? 32 : NW * IPW / P;
  const int sub = blockIdx.x, n0 = sub * R;
  // x is read by a full gate and by the up products of the partial-row and
  // chunk modes; a low-rank split-mode or pack-only gate leaves it out of LDS
  const bool need_x = dec_gate_needs_x(LOWRANK, MODE, d.up);
  uint16_t* s_x = reinterpret_cast<uint16_t*>(s_dyn);                               // [MAXM x d] bf16
  float* s_t = reinterpret_cast<float*>(reinterpret_cast<char*>(s_dyn) + (need_x ? (size_t)MAXM * dm * 2 : 0));  // [MAXM x rank]

  // ---- gate row loads first; the token inputs are staged while they fly
  // 5..16 tokens, low rank, 32-row sub-tiles over a K of 512: the gate on
  // matrix cores (t split into bf16 hi + lo); otherwise the VALU GEMV (at 2..4
  // tokens it is as fast, with fewer barriers)
  constexpr bool MF = LOWRANK && MAXM >= 8 && NW == 8;
  // K = 512 (16 steps) over the waves of a row group: 32-row sub-tiles (two
  // groups of four waves, 4 steps each) or, with IPW = 8, 64-row sub-tiles
  // (four groups of two waves, 8 steps each)
  constexpr int MF_NG = IPW == 8 ? 4 : 2;
  constexpr int MF_DS = 16 / (NW / MF_NG);
  const bool use_mf = MF && R == 16 * MF_NG && K == 512;
  const bool use_fg = FG && R == 32 && K % 128 == 0 && K <= 128 * kFgMaxSteps;
  uint4 a[IPW];
  uint4 am[MF ? MF_DS : 1];
  uint4 af[FG ? kFgMaxSteps : 1];
  if constexpr (MF) {
    if (use_mf) dec_mfma_issue<8, MF_NG, MF_DS>(reinterpret_cast<const uint16_t*>(d.a_gate), K, n0, am);
    else if constexpr (IPW <= 4) dec_gemv_issue<NW, IPW>(reinterpret_cast<const uint16_t*>(d.a_gate), F, K, P, n0, a);
  } else if constexpr (FG) {
    if (use_fg) dec_fg_issue(reinterpret_cast<const uint16_t*>(d.a_gate), K, n0, af);
    else dec_gemv_issue<NW, IPW>(reinterpret_cast<const uint16_t*>(d.a_gate), F, K, P, n0, a);
  } else {
    dec_gemv_issue<NW, IPW>(reinterpret_cast<const uint16_t*>(d.a_gate), F, K, P, n0, a);
  }
  if (need_x) stage_rows<MAXM>(s_dyn, reinterpret_cast<const uint4*>(d.x), M, dm / 8, dm / 8);
  if (LOWRANK) {
    if (d.nslab > 0) {
      // t = the first stage's slabs, added in slab order
      const int c4 = d.rank / 4;
      constexpr int NP = MAXM >= 16 ? 1 : 2;          // chunks per thread in flight, 8 slab loads each
      for (int base = threadIdx.x; base < MAXM * c4; base += NP * blockDim.x) {
        float4 v[NP][8];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int p = base + i * blockDim.x, m = p / c4, c = p - m * c4;
#pragma unroll
          for (int z = 0; z < 8; ++z)
            v[i][z] = (p < MAXM * c4 && m < M && z < d.nslab)
                          ? *reinterpret_cast<const float4*>(d.tslab + ((size_t)z * M + m) * d.rank + c * 4)
                          : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int p = base + i * blockDim.x;
          float4 acc = v[i][0];
#pragma unroll
          for (int z = 1; z < 8; ++z) {
            acc.x += v[i][z].x;
            acc.y += v[i][z].y;
            acc.z += v[i][z].z;
            acc.w += v[i][z].w;
          }
          if (p < MAXM * c4) reinterpret_cast<float4*>(s_t)[p] = acc;
        }
      }
    } else {
      stage_rows<MAXM>(reinterpret_cast<uint4*>(s_t), reinterpret_cast<const uint4*>(d.t), M, d.rank / 4, d.rank / 4);
    }
  }
  const uint32_t epoch = __hip_atomic_load(&d.ctrl[CTRL_EPOCH], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const WaitCtl wc = wait_ctl(d.ctrl, epoch);
  __syncthreads();
  if constexpr (MF) {
    if (use_mf) dec_mfma_finish<8, MF_NG, MF_DS, MAXM>(am, K, s_t, M, s_acc, s_g);
    else if constexpr (IPW <= 4) dec_gemv_finish<NW, IPW, MAXM, LOWRANK>(a, K, P, s_x, s_t, s_part, s_g);
  } else if constexpr (FG) {
    if (use_fg) dec_fg_finish<MAXM>(af, K, s_x, M, s_acc, s_g);
    else dec_gemv_finish<NW, IPW, MAXM, LOWRANK>(a, K, P, s_x, s_t, s_part, s_g);
  } else {
    dec_gemv_finish<NW, IPW, MAXM, LOWRANK>(a, K, P, s_x, s_t, s_part, s_g);
  }

  // ---- selection: one wave per token; the sub-tile's mask is one ballot (R <= 64)
  constexpr bool ONE = MAXM == 1 && MODE != DEC_SPLIT;
  const int T = d.T, Q = T / R, q = (n0 % T) / R, j = n0 / T;
  const int ntiles = F / T, nsub = F / R;
  for (int m = wave; m < M; m += NW) {             // one wave per token (two at 16 tokens)
    const float b = dec_bias(d, m), cut = dec_cut(d, m);
    bool act = false;
    if (lane < R) {
      const float g = s_g[lane * MAXM + m];
      if (d.g_debug) d.g_debug[(size_t)m * F + n0 + lane] = g;
      act = (g + b) > cut;
    }
    const uint64_t bal = ballot64(act);
    if (lane == 0) {
      s_bal[m] = bal;
      if (Q > 1)
        store64_relaxed(d.lb + (size_t)m * nsub + sub, ((uint64_t)epoch << 32) | (uint32_t)__popcll(bal));
    }
    if constexpr (ONE) {
      // one token: the union is this ballot, and its row list is written
      // before the barrier that publishes the ballot
      if (d.up) {
        if ((bal >> lane) & 1ull) s_urow[__popcll(bal & lanemask_lt())] = lane;
        if (lane == 0) d.umask[sub] = bal;
      }
    }
    if constexpr (MAXM <= 8) break;                   // at most one token a wave
  }
  if ((int)threadIdx.x < MAXM && (int)threadIdx.x >= M) s_bal[threadIdx.x] = 0ull;
  __syncthreads();

  // first read of the earlier sub-tiles' counts of tile j (per token), while
  // this workgroup's up products run
  const bool tok_wave = wave < M && Q > 1;
  const uint64_t* twp = d.lb + (size_t)(tok_wave ? wave : 0) * nsub + (size_t)j * Q + lane;
  uint64_t tw = 0;
  if (tok_wave && lane < q) tw = load64_relaxed(twp);

  // TwELL pack of token m: this sub-tile's entries at their offset inside
  // tile j (wave-wide: one lane per row of the sub-tile)
  auto write_pack = [&](int m) {
    const uint64_t bal = s_bal[m];
    int pre = 0;
    if (Q > 1) {
      // the wave's first token's first read was issued early
      const uint64_t* wp = d.lb + (size_t)m * nsub + (size_t)j * Q + lane;
      const uint64_t first = m == wave ? tw : (lane < q ? load64_relaxed(wp) : 0ull);
      pre = wave_sum_i(lane < q ? lb_count(wp, wc, first, d.ctrl) : 0);
    }
    const size_t slot0 = ((size_t)m * ntiles + j) * d.E;
    const bool act = (bal >> lane) & 1ull;
    const int pos = pre + __popcll(bal & lanemask_lt());
    if (act && pos < d.E) {
      d.idx[slot0 + pos] = (uint16_t)(q * R + lane);
      const float z = s_g[lane * MAXM + m] + dec_bias(d, m);
      reinterpret_cast<uint16_t*>(d.val)[slot0 + pos] = (uint16_t)f2bf(z);
    }
    if (q == Q - 1) {
      const int total = pre + __popcll(bal);
      if (lane == 0) d.cnt[(size_t)m * ntiles + j] = total;
      for (int s = min(total, d.E) + lane; s < d.E; s += 64) {
        d.idx[slot0 + s] = 0xFFFF;
        reinterpret_cast<uint16_t*>(d.val)[slot0 + s] = 0;
      }
    }
  };
  // one token, partial rows: wave 0 writes the pack while the first batch's
  // row loads are in flight (the up rows go to waves 1.., wave 0 last)
  bool packed = false;

  // ---- up products of the neurons active for any token: h = a * <W_up[i,:], x>
  if (d.up) {
    uint64_t uni = 0ull;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) uni |= s_bal[m];
    const int nu = __popcll(uni);
    if constexpr (!ONE) {
      if (threadIdx.x == 0) d.umask[sub] = uni;
      if (MODE == DEC_SPLIT) {
        // split mode: the activations of the union neurons for k_dec_up
        for (int p = threadIdx.x; p < R * MAXM; p += NW * 64) {
          const int r = p / MAXM, m = p % MAXM;
          if (m < M && ((uni >> r) & 1ull)) {
            const bool on = (s_bal[m] >> r) & 1ull;
            d.ad[(size_t)m * F + n0 + r] = on ? s_g[r * MAXM + m] + dec_bias(d, m) : 0.f;
          }
        }
      }
      if (wave == 0 && ((uni >> lane) & 1ull)) s_urow[__popcll(uni & lanemask_lt())] = lane;
      __syncthreads();
    }
    const int pd = (dm + 511) / 512;
    // one up product: the owner wave reads W_up[n, :] (8 KB at d = 4096) and
    // reduces the dot with every token across its lanes
    auto up_row = [&](int k, bool to_lds) {
      const int r = s_urow[k], n = n0 + r;
      const uint16_t* row = reinterpret_cast<const uint16_t*>(d.w_up) + (size_t)n * dm;
      uint4 w[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = c * 512 + lane * 8;
        w[c] = (c < pd && col < dm) ? ldg16(row + col) : uint4{0, 0, 0, 0};
      }
      float v[MAXM];
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int col = c * 512 + lane * 8;
          if (c < pd && col < dm) s = dot8_bf(w[c], *reinterpret_cast<const uint4*>(s_x + (size_t)m * dm + col), s);
        }
        v[m] = s;
      }
      WaveTRed<MAXM, 32>::run(v, lane);
      constexpr int SH = 6 - Log2<MAXM>::value;
      if ((lane & ((1 << SH) - 1)) == 0) {
        const int m = lane >> SH;
        if (m < M) {
          const bool on = (s_bal[m] >> r) & 1ull;
          const float av = on ? s_g[r * MAXM + m] + dec_bias(d, m) : 0.f;
          if (to_lds) s_h[k * MAXM + m] = av * v[0];
          else d.hd[(size_t)m * F + n] = av * v[0];
        }
      }
    };
    if (MODE == DEC_CHUNK) {
      for (int k = wave; k < nu; k += NW) up_row(k, false);
    } else if (MODE == DEC_PART) {
      // partial-row mode: every thread owns CPT consecutive columns of y; the
      // down rows of a batch of entries are loaded (coalesced, 8 or 16 bytes
      // per thread) in the same round as their up rows, then scaled by h and
      // summed in entry order
      constexpr int CPT = NW == 16 ? 4 : 8;             // 64 * NW * CPT = 4096 columns
      constexpr int DB = MAXM == 1 ? 16 : (MAXM == 2 ? 8 : 4);
      using DV = typename std::conditional<CPT == 4, uint2, uint4>::type;
      const bool colt = (int)threadIdx.x * CPT < dm;
      const uint16_t* wdn = reinterpret_cast<const uint16_t*>(d.w_down_nm) + (size_t)threadIdx.x * CPT;
      float acc[MAXM][CPT];
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
#pragma unroll
        for (int q = 0; q < CPT; ++q) acc[m][q] = 0.f;
      for (int k0 = 0; k0 < nu; k0 += DB) {
        DV dw[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) {
          const int k = k0 + i;
          dw[i] = (k < nu && colt) ? *reinterpret_cast<const DV*>(wdn + (size_t)(n0 + s_urow[k]) * dm) : DV{};
        }
        if constexpr (ONE) {
          if (k0 == 0 && wave == 0) write_pack(0);
          for (int k = k0 + (wave + NW - 1) % NW; k < min(nu, k0 + DB); k += NW) up_row(k, true);
        } else {
          for (int k = k0 + wave; k < min(nu, k0 + DB); k += NW) up_row(k, true);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < DB; ++i) {
          const int k = k0 + i;
          if (k < nu) {
            float f[CPT];
            const uint32_t* wv = reinterpret_cast<const uint32_t*>(&dw[i]);
#pragma unroll
            for (int q = 0; q < CPT / 2; ++q) {
              f[2 * q] = __uint_as_float(wv[q] << 16);
              f[2 * q + 1] = __uint_as_float(wv[q] & 0xFFFF0000u);
            }
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
              const float hv = s_h[k * MAXM + m];
#pragma unroll
              for (int q = 0; q < CPT; ++q) acc[m][q] = fmaf(hv, f[q], acc[m][q]);
            }
          }
        }
        __syncthreads();                                // s_h is rewritten by the next batch
      }
      if (ONE && nu > 0) packed = true;
      if (nu > 0 && colt) {
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
          if (m < M) {
            float* dst = d.part + ((size_t)sub * M + m) * dm + threadIdx.x * CPT;
#pragma unroll
            for (int q = 0; q < CPT; q += 4)
              *reinterpret_cast<float4*>(dst + q) = float4{acc[m][q], acc[m][q + 1], acc[m][q + 2], acc[m][q + 3]};
          }
      }
    }
  }

  // ---- TwELL pack (unless written during the up and down loads above)
  if (!packed) {
    for (int m = wave; m < M; m += NW) {
      write_pack(m);
      if constexpr (MAXM <= 8) break;                 // at most one token a wave
    }
  }
}
template <int NW, int IPW, int MAXM, bool LOWRANK, int MODE>
__global__ __launch_bounds__(64 * NW) void k_dec_gate(const DecodeDesc d) { dec_gate_body<NW, IPW, MAXM, LOWRANK, MODE>(d); }
template <int NW, int IPW, int MAXM, bool LOWRANK, int MODE>
__global__ __launch_bounds__(64 * NW) void k_dec_gate_grp(const DecGroup g) { dec_gate_body<NW, IPW, MAXM, LOWRANK, MODE>(g.d[blockIdx.y]); }

// ------------------------------------------------------------------ k_dec_down
constexpr int kDownThreads = 256;
constexpr int kDecMaxSub = 2048;                      // sub-tiles the down kernel's LDS holds

// position of the k-th (from 0) set bit of w (k < popcount(w))
__device__ __forceinline__ int nth_set_bit(uint64_t w, int k) {
  int pos = 0;
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const int c = __popcll(w & ((1ull << half) - 1ull));
    if (k >= c) {
      k -= c;
      w >>= half;
      pos += half;
    }
  }
  return pos;
}

template <int MAXM>
__global__ __launch_bounds__(kDownThreads) void k_dec_down(const DecodeDesc d) {
  constexpr int B = MAXM <= 4 ? 8 : 4;               // entries in flight per thread
  __shared__ uint64_t s_mask[kDecMaxSub];
  __shared__ int s_pre[kDecMaxSub + 1];
  __shared__ int s_scan[kDownThreads / 64];
  __shared__ float s_red[kDownThreads / 64][8 * MAXM];
  const int nch = d.d / 8;
  if (d.route_pass && (int)blockIdx.x == nch) {
    route_pass(d.route);
    return;
  }
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int b = blockIdx.x;
  const int c = (b & 7) * (nch >> 3) + (b >> 3);       // chunks of one 128-byte line share an XCD
  const int F = d.F, M = d.M, R = d.R, nsub = F / R;

  // union masks of a contiguous run of sub-tiles per thread, and the
  // exclusive prefix of their popcounts
  const int per = (nsub + kDownThreads - 1) / kDownThreads;
  const int s0 = min(nsub, tid * per), s1 = min(nsub, s0 + per);
  int loc = 0;
  for (int s = s0; s < s1; ++s) {
    const uint64_t w = d.umask[s];
    s_mask[s] = w;
    loc += __popcll(w);
  }
  int total;
  int run = block_excl_scan<kDownThreads>(loc, s_scan, &total);
  for (int s = s0; s < s1; ++s) {
    s_pre[s] = run;
    run += __popcll(s_mask[s]);
  }
  __syncthreads();

  float acc[MAXM][8];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[m][k] = 0.f;
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(d.w_down_nm) + (size_t)c * 8;
  for (int e0 = tid; e0 < total; e0 += kDownThreads * B) {
    uint4 w[B];
    float h[B][MAXM];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int e = e0 + i * kDownThreads;
      w[i] = uint4{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < MAXM; ++m) h[i][m] = 0.f;
      if (e < total) {
        int lo = 0, hi = nsub - 1;                     // last sub-tile with s_pre <= e
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pre[mid] <= e) lo = mid;
          else hi = mid - 1;
        }
        const int n = lo * R + nth_set_bit(s_mask[lo], e - s_pre[lo]);
        w[i] = ldg16(wd + (size_t)n * d.d);
#pragma unroll
        for (int m = 0; m < MAXM; ++m) h[i][m] = m < M ? d.hd[(size_t)m * F + n] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      float f[8];
      unpack8(w[i], f);
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[m][k] = fmaf(h[i][m], f[k], acc[m][k]);
    }
  }

  // reduce the 8 * MAXM sums over the workgroup in a fixed order
  constexpr int V = 8 * MAXM;
  float v[V];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[m * 8 + k] = acc[m][k];
  WaveTRed<V, 32>::run(v, lane);
  constexpr int SH = 6 - Log2<V>::value;
  if ((lane & ((1 << SH) - 1)) == 0) s_red[wave][lane >> SH] = v[0];
  __syncthreads();
  if (tid < V) {
    const int m = tid / 8, k = tid % 8;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kDownThreads / 64; ++w) s += s_red[w][tid];
    if (m < M) reinterpret_cast<uint16_t*>(d.y)[(size_t)m * d.d + c * 8 + k] = (uint16_t)f2bf(s);
  }
}

// ------------------------------------------------------------------ k_dec_reduce
// y[m, slice] = sum over the non-empty sub-tiles (ascending) of their partial
// rows. A workgroup owns a 128-byte slice (32 fp32 columns) of every token's
// row: 8 threads read one partial row's slice (16 bytes each); thread row r
// takes the sub-tiles r, r + 32, r + 64, .. and adds the non-empty ones in
// that order, and the 32 thread-row sums per column are then added in order.
// (Loading every sub-tile's row beside its mask, one memory round instead of
// two, measured the same.)
constexpr int kRedThreads = 256;

template <int MAXM>
__device__ __forceinline__ void dec_reduce_body(const DecodeDesc& d) {
  constexpr int B = 16 / MAXM;                          // sub-tiles in flight per thread
  __shared__ float s_red[MAXM][32][33];
  const int nsl = d.d / 32;
  if (d.route_pass && (int)blockIdx.x == nsl) {
    route_pass(d.route);
    return;
  }
  const int tid = threadIdx.x, q = tid & 7, r = tid >> 3;
  const int sl = blockIdx.x, M = d.M, dm = d.d, nsub = d.F / d.R;
  float acc[MAXM][4];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[m][k] = 0.f;
  const size_t col = (size_t)sl * 32 + q * 4;
  for (int s0 = r; s0 < nsub; s0 += 32 * B) {
    uint64_t w[B];
    float4 v[B][MAXM];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = d.umask[min(s0 + 32 * i, nsub - 1)];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int sv = s0 + 32 * i;
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        v[i][m] = (sv < nsub && w[i] != 0ull && m < M)
                      ? *reinterpret_cast<const float4*>(d.part + ((size_t)sv * M + m) * dm + col)
                      : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < B; ++i)
      if (s0 + 32 * i < nsub && w[i] != 0ull) {
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
          acc[m][0] += v[i][m].x;
          acc[m][1] += v[i][m].y;
          acc[m][2] += v[i][m].z;
          acc[m][3] += v[i][m].w;
        }
      }
  }
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k) s_red[m][q * 4 + k][r] = acc[m][k];
  __syncthreads();
  for (int o = tid; o < MAXM * 32; o += kRedThreads) {
    const int m = o / 32, c = o % 32;
    float sum = 0.f;
#pragma unroll 8
    for (int rr = 0; rr < 32; ++rr) sum += s_red[m][c][rr];
    if (m < M) reinterpret_cast<uint16_t*>(d.y)[(size_t)m * dm + (size_t)sl * 32 + c] = (uint16_t)f2bf(sum);
  }
}
template <int MAXM>
__global__ __launch_bounds__(kRedThreads) void k_dec_reduce(const DecodeDesc d) { dec_reduce_body<MAXM>(d); }
template <int MAXM>
__global__ __launch_bounds__(kRedThreads) void k_dec_reduce_grp(const DecGroup g) { dec_reduce_body<MAXM>(g.d[blockIdx.y]); }

// ------------------------------------------------------------------ k_dec_up (split mode)
// The union neurons (set bits of the sub-tile masks, ascending) form the list;
// workgroup b of the G in the grid takes the list entries [b U / G,
// (b + 1) U / G) (U the list length), so every workgroup streams the same
// number of W_up rows. Its entries form up to three groups of 16 rows whose
// up products are a small dense contraction, 16 rows x d by d x M tokens, on
// v_mfma_f32_16x16x32_bf16: wave w owns the contiguous eighth of d, step j of
// it covering 32 elements. Operand lane l holds row l % 16 at the 16-byte
// chunk 4 j + l / 16, so one load instruction reads 64 contiguous bytes of each
// of the 16 rows and two consecutive steps a whole 128-byte line; all loads of
// the workgroup's groups are issued before the first product. The tokens' x
// (B operand) sits in LDS, one row per token padded by 16 bytes so that the
// eight tokens of a read fall in distinct banks. The eight waves' partial
// 16 x 16 tiles are summed in LDS in wave order; h = a * u is stored as bf16 in
// token-major rows hT[token][entry], the neuron ids in the list. The last
// workgroup zeroes the entries from U up to the next multiple of 32, which the
// down kernel reads whole.
constexpr int kUpWaves = 8;
constexpr int kUpGrid = 256;
constexpr int kUpMaxSteps = 16;                        // 32-element steps per wave (d <= 4096)
constexpr int kUpNB = 3;                               // groups of 16 entries in flight
constexpr int kUpMaxEnt = 128;                         // entries per workgroup (F <= 128 * kUpGrid)
// id slots: the group loop reads kUpNB groups of 16 at a time, so the slots
// run to the next multiple of 16 * kUpNB; slots from the workgroup's entry
// count on hold -1 (no row)
constexpr int kUpNrnSlots = (kUpMaxEnt + 16 * kUpNB - 1) / (16 * kUpNB) * (16 * kUpNB);

__device__ __forceinline__ void dec_up_body(const DecodeDesc& d) {
  extern __shared__ uint4 s_dyn[];                     // x: M rows of d + 8 bf16; masks; prefixes
  __shared__ int s_scan[kUpWaves];
  __shared__ int s_nrn[kUpNrnSlots];
  __shared__ f32x4_t s_acc[kUpWaves][kUpNB][64];
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int M = d.M, dm = d.d, F = d.F, R = d.R, nsub = F / R;
  const int G = gridDim.x, b = blockIdx.x;
  const int steps = dm / (32 * kUpWaves);              // per wave
  const int q = lane >> 4, r16 = lane & 15;
  const int k0 = wave * steps * 32;                    // first element of the wave's K range
  const int ldx = dm + 8;                              // LDS row stride of x (elements)
  constexpr int NT = 64 * kUpWaves;
  // the sub-tile masks and their prefixes follow x (nsub entries each)
  uint64_t* s_mask = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(s_dyn) + (size_t)M * ldx * 2);
  int* s_pre = reinterpret_cast<int*>(s_mask + nsub);

  // masks and their prefix; x into LDS
  const int per = (nsub + NT - 1) / NT;                 // sub-tiles per thread (<= 4)
  const int s0 = min(nsub, tid * per), s1 = min(nsub, s0 + per);
  // the masks' loads and x's go out together (one memory round trip)
  uint64_t mw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mw[i] = d.umask[min(s0 + i, nsub - 1)];
  {
    uint16_t* sx = reinterpret_cast<uint16_t*>(s_dyn);
    const int c16 = dm / 8;
    // M * d / 8 <= 16 * NT (d <= 4096, M <= 16): one unrolled round, the
    // guards uniform across the block
    const int n = M * c16;
    uint4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (u * NT < n) v[u] = ldg16(reinterpret_cast<const uint16_t*>(d.x) + (size_t)min(tid + u * NT, n - 1) * 8);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int p = tid + u * NT, m = p / c16, c = p - m * c16;
      if (u * NT < n && p < n) *reinterpret_cast<uint4*>(sx + (size_t)m * ldx + c * 8) = v[u];
    }
  }
  int loc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (s0 + i < s1) {
      s_mask[s0 + i] = mw[i];
      loc += __popcll(mw[i]);
    }
  int total;
  int run = block_excl_scan<NT>(loc, s_scan, &total);
  for (int s = s0; s < s1; ++s) {
    s_pre[s] = run;
    run += __popcll(s_mask[s]);
  }
  __syncthreads();
  if (b == 0 && tid == 0) *d.ul_total = total;
  const int e0 = (int)((long long)total * b / G), e1 = (int)((long long)total * (b + 1) / G);
  const int ne = e1 - e0;
  for (int i = tid; i < kUpNrnSlots; i += NT) {
    int n = -1;
    if (i < ne) {
      const int e = e0 + i;
      int lo = 0, hi = nsub - 1;                         // last sub-tile with s_pre <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= e) lo = mid;
        else hi = mid - 1;
      }
      n = lo * R + nth_set_bit(s_mask[lo], e - s_pre[lo]);
    }
    s_nrn[i] = n;
  }
  // the pad entries [total, total rounded up to 32)
  if (b == G - 1) {
    const int pad = (total + 31) / 32 * 32;
    uint16_t* hT = reinterpret_cast<uint16_t*>(d.ul_h);
    for (int p = tid; p < (pad - total) * M; p += NT) {
      const int m = p / (pad - total), e = total + p % (pad - total);
      hT[(size_t)m * d.ldh + e] = 0;
      if (m == 0) d.ul_nrn[e] = 0;
    }
  }
  __syncthreads();

  const uint16_t* sx = reinterpret_cast<const uint16_t*>(s_dyn);
  uint16_t* hT = reinterpret_cast<uint16_t*>(d.ul_h);
  for (int g0 = 0; g0 * 16 < ne; g0 += kUpNB) {
    uint4 aw[kUpNB][kUpMaxSteps];
#pragma unroll
    for (int g = 0; g < kUpNB; ++g) {
      const int nrn = s_nrn[(g0 + g) * 16 + r16];
#pragma unroll
      for (int j = 0; j < kUpMaxSteps; ++j) aw[g][j] = uint4{0, 0, 0, 0};
      if (nrn >= 0) {
        const uint16_t* wr = reinterpret_cast<const uint16_t*>(d.w_up) + (size_t)nrn * dm + k0 + q * 8;
#pragma unroll
        for (int j = 0; j < kUpMaxSteps; ++j)
          if (j < steps) aw[g][j] = ldg16(wr + j * 32);
      }
    }
    // activations a[token][neuron] of the entries wave g reduces
    float av[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave < kUpNB && r16 < M) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = s_nrn[(g0 + wave) * 16 + 4 * q + v];
        if (n >= 0) av[v] = d.ad[(size_t)r16 * F + n];
      }
    }
    f32x4_t acc[kUpNB];
#pragma unroll
    for (int g = 0; g < kUpNB; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* xr = sx + (size_t)min(r16, M - 1) * ldx + k0 + q * 8;
#pragma unroll
    for (int j = 0; j < kUpMaxSteps; ++j) {
      if (j < steps) {
        uint4 bx = *reinterpret_cast<const uint4*>(xr + j * 32);
        if (r16 >= M) bx = uint4{0, 0, 0, 0};
#pragma unroll
        for (int g = 0; g < kUpNB; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(aw[g][j]), as_bf16x8(bx), acc[g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int g = 0; g < kUpNB; ++g) s_acc[wave][g][lane] = acc[g];
    __syncthreads();
    if (wave < kUpNB && (g0 + wave) * 16 < ne) {
      const int g = wave;
      f32x4_t u = s_acc[0][g][lane];
#pragma unroll
      for (int w = 1; w < kUpWaves; ++w) {
        const f32x4_t t = s_acc[w][g][lane];
        u[0] += t[0];
        u[1] += t[1];
        u[2] += t[2];
        u[3] += t[3];
      }
      // lane l: local entries 16 (g0 + g) + 4 (l / 16) + v, token l % 16
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = (g0 + g) * 16 + 4 * q + v;
        if (i < ne) {
          if (r16 < M) hT[(size_t)r16 * d.ldh + e0 + i] = (uint16_t)f2bf(av[v] * u[v]);
          if (r16 == 0) d.ul_nrn[e0 + i] = s_nrn[i];
        }
      }
    }
    __syncthreads();
  }
}
__global__ __launch_bounds__(64 * kUpWaves) void k_dec_up(const DecodeDesc d) { dec_up_body(d); }
__global__ __launch_bounds__(64 * kUpWaves) void k_dec_up_grp(const DecGroup g) { dec_up_body(g.d[blockIdx.y]); }

// ------------------------------------------------------------------ k_dec_down2 (split mode)
// y[token, :] = sum over the list of h[token, e] W_down[:, n_e], as MFMA tiles
// D[column][token] += W_down^T[column][e] hT[token][e] over 32 entries a step.
// A workgroup owns a 64-column slice of y and one of S contiguous ranges of
// 32-entry blocks; its four waves take the blocks in turn. A wave gathers the
// block's 32 row slices (128 bytes each: eight lanes per row, whole lines)
// into its own LDS tile and reads them back transposed as the A operand
// (lane l: column l % 16 of a 16-column block, entries 8 (l / 16) .. + 7) with
// ds_read_b64_tr_b16: in each 16-lane group, output lane j receives element
// j % 4 of the 8 bytes source lane 4 v + j / 4 addressed, as its value v. So
// source lane 4 v + u of group q points at row 8 q + 4 h + v, columns
// c0 + 4 u .. + 3, and two reads (h = 0, 1) give a lane its column's 8 rows.
// The 16-byte chunks of a row are stored XOR-swizzled by 2 (row % 4), which
// spreads the 16 rows one read touches evenly over the banks. The B operand
// is read straight from hT (16 bytes a lane). The four
// waves' tiles are summed in LDS in wave order and written as the group's
// partial rows; k_dec_reduce2 adds the S groups in group order.
constexpr int kDown2Threads = 256;
constexpr int kDown2MaxIds = 2048;                     // list entries per workgroup

__device__ __forceinline__ int dn_slot(int row, int c) { return row * 8 + (c ^ ((row & 3) << 1)); }
typedef short dn_v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dec_down2_body(const DecodeDesc& d) {
  constexpr int NW = kDown2Threads / 64;
  __shared__ uint4 s_w[NW][2][32 * 8];                 // per wave: two blocks of 32 rows x 128 bytes
  __shared__ int s_ids[kDown2MaxIds];
  __shared__ f32x4_t s_acc[NW][4][64];
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int S = d.ngroups, nsl = d.d / 64;
  const int sl = blockIdx.x % nsl, g = blockIdx.x / nsl;
  const int M = d.M, dm = d.d, ldh = d.ldh;
  const int total = *d.ul_total;
  const int nkb = (total + 31) / 32;
  const int kb0 = (int)((long long)nkb * g / S), kb1 = (int)((long long)nkb * (g + 1) / S);
  for (int i = tid; i < (kb1 - kb0) * 32; i += kDown2Threads) s_ids[i] = d.ul_nrn[kb0 * 32 + i];
  __syncthreads();
  const int q = lane >> 4, r16 = lane & 15;
  const int lrow = lane >> 3, lch = lane & 7;          // gather: row lrow + 8 i, chunk lch
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(d.w_down_nm) + (size_t)sl * 64 + lch * 8;
  const uint16_t* hT = reinterpret_cast<const uint16_t*>(d.ul_h);
  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // transposed-read source of this lane: row 8 q + 4 h + r16 / 4, columns 4 (r16 % 4) .. + 3
  const int trow = 8 * q + (r16 >> 2), tcol = 4 * (r16 & 3);
  for (int kb = kb0 + wave; kb < kb1; kb += 2 * NW) {
    const int kbb = kb + NW;
    const bool two = kbb < kb1;
    uint4 w[2][4];
    uint4 hb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = u ? kbb : kb;
      const bool on = u == 0 || two;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = on ? s_ids[(kk - kb0) * 32 + lrow + 8 * i] : 0;
        w[u][i] = on ? ldg16(wd + (size_t)n * dm) : uint4{0, 0, 0, 0};
      }
      hb[u] = (on && r16 < M) ? ldg16(hT + (size_t)r16 * ldh + kk * 32 + q * 8) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_w[wave][u][dn_slot(lrow + 8 * i, lch)] = w[u][i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
      const uint16_t* tb = reinterpret_cast<const uint16_t*>(&s_w[wave][u][0]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // columns 16 c + tcol .. + 3 lie in chunk 2 c + tcol / 8 at element tcol % 8
        const int ch = 2 * c + (tcol >> 3), el = tcol & 7;
        const dn_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) dn_v4s*)(tb + dn_slot(trow, ch) * 8 + el));
        const dn_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) dn_v4s*)(tb + dn_slot(trow + 4, ch) * 8 + el));
        const uint4 a = uint4{(uint32_t)(uint16_t)lo.x | ((uint32_t)(uint16_t)lo.y << 16),
                              (uint32_t)(uint16_t)lo.z | ((uint32_t)(uint16_t)lo.w << 16),
                              (uint32_t)(uint16_t)hi.x | ((uint32_t)(uint16_t)hi.y << 16),
                              (uint32_t)(uint16_t)hi.z | ((uint32_t)(uint16_t)hi.w << 16)};
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(hb[u]), acc[c], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) s_acc[wave][c][lane] = acc[c];
  __syncthreads();
  {
    const int c = tid >> 6, l = tid & 63;              // 256 threads: 4 column blocks x 64 lanes
    f32x4_t s = s_acc[0][c][l];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) {
      const f32x4_t t = s_acc[w2][c][l];
      s[0] += t[0];
      s[1] += t[1];
      s[2] += t[2];
      s[3] += t[3];
    }
    // lane l: columns 16 c + 4 (l / 16) + v, token l % 16
    const int tok = l & 15;
    if (tok < M)
      *reinterpret_cast<float4*>(d.part + ((size_t)g * M + tok) * dm + sl * 64 + 16 * c + 4 * (l >> 4)) =
          float4{s[0], s[1], s[2], s[3]};
  }
}
__global__ __launch_bounds__(kDown2Threads) void k_dec_down2(const DecodeDesc d) { dec_down2_body(d); }
__global__ __launch_bounds__(kDown2Threads) void k_dec_down2_grp(const DecGroup g) { dec_down2_body(g.d[blockIdx.y]); }

// y = sum of the S group partials in group order; the extra last workgroup
// routes the pack.
__device__ __forceinline__ void dec_reduce2_body(const DecodeDesc& d) {
  const int n = d.M * d.d;
  if (d.route_pass && (int)blockIdx.x == (n + 1023) / 1024) {
    route_pass(d.route);
    return;
  }
  const int i0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= n) return;
  float4 acc = float4{0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < d.ngroups; ++g) {
    const float4 p = *reinterpret_cast<const float4*>(d.part + (size_t)g * n + i0);
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  uint16_t* y = reinterpret_cast<uint16_t*>(d.y) + i0;
  *reinterpret_cast<uint2*>(y) = uint2{f2bf(acc.x) | (f2bf(acc.y) << 16), f2bf(acc.z) | (f2bf(acc.w) << 16)};
}
__global__ __launch_bounds__(256) void k_dec_reduce2(const DecodeDesc d) { dec_reduce2_body(d); }
__global__ __launch_bounds__(256) void k_dec_reduce2_grp(const DecGroup g) { dec_reduce2_body(g.d[blockIdx.y]); }

// ------------------------------------------------------------------ launches
static int pow2_pieces(int K) {
  int P = 1;
  while (P * 512 < K) P <<= 1;
  return P;
}

static int dec_maxm(int M) { return M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 8 : 16))); }

size_t dec_lowrank_lds(const DecodeDesc& d) { return (size_t)dec_maxm(d.M) * d.d * 2; }
// The gate kernel's mode: the split sequence from 9 tokens, the chunk-mode
// kernel for a pack-only pass, otherwise the planned mode.
static int dec_gate_mode(const DecodeDesc& d) {
  if (dec_maxm(d.M) == 16) return DEC_SPLIT;
  return d.up ? d.mode : DEC_CHUNK;
}

size_t dec_gate_lds(const DecodeDesc& d) {
  const size_t mx = dec_maxm(d.M);
  return (dec_gate_needs_x(d.rank > 0, dec_gate_mode(d), d.up) ? mx * d.d * 2 : 0) +
         (d.rank ? mx * d.rank * 4 : 0);
}

template <typename Kern>
static hipError_t lds_attr(Kern k, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int IPW, int MAXM>
static hipError_t go_lowrank(const DecodeDesc& d, hipStream_t s) {
  const int P = d.ipw, R = kDecVWaves * IPW / P;
  const size_t lds = dec_lowrank_lds(d);
  hipError_t e = lds_attr(k_dec_lowrank<IPW, MAXM>, lds);
  if (e != hipSuccess) return e;
  ffn_launch((k_dec_lowrank<IPW, MAXM>), dim3((d.rank + R - 1) / R), dim3(64 * kDecVWaves), lds, s, d);
  return hipGetLastError();
}

// d.ipw carries the pieces per V row here; IPW is chosen so that a workgroup
// covers whole rows: R = 4 * IPW / P >= 1.
template <int MAXM>
static hipError_t go_lowrank_m(const DecodeDesc& d, hipStream_t s) {
  if (d.ipw >= 8) return go_lowrank<4, MAXM>(d, s);    // P = 8: 2 rows per workgroup
  if (d.ipw == 4) return go_lowrank<2, MAXM>(d, s);    // P = 4: 2 rows
  return go_lowrank<2, MAXM>(d, s);                    // P <= 2: 4 or 8 rows
}

hipError_t launch_dec_lowrank(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || d.rank <= 0) return hipErrorInvalidValue;
  // several tokens: the matrix-core kernel, writing nslab slabs
  if (d.nslab > 0) {
    const int nwv = d.nslab >= 1 && d.nslab <= 8 ? lowrank_mf_waves(d.d, d.nslab) : 0;
    if (nwv == 0 || d.M < 2 || d.rank % 16 != 0 || !d.tslab) return hipErrorInvalidValue;
    ffn_launch(k_dec_lowrank_mf, dim3(d.rank / 16, d.nslab), dim3(64 * nwv), 0, s, d);
    return hipGetLastError();
  }
  DecodeDesc e = d;
  e.ipw = pow2_pieces(d.d);
  if (e.ipw > 8) return hipErrorInvalidValue;
  if (d.M > 8) return hipErrorInvalidValue;            // 9..16 tokens: the matrix-core kernel only
  switch (dec_maxm(d.M)) {
    case 1: return go_lowrank_m<1>(e, s);
    case 2: return go_lowrank_m<2>(e, s);
    case 4: return go_lowrank_m<4>(e, s);
    default: return go_lowrank_m<8>(e, s);
  }
}

template <int IPW, int MAXM, bool LOWRANK, int MODE>
static hipError_t go_gate_k(const DecodeDesc& d, hipStream_t s) {
  constexpr int NW = dec_gate_waves(MAXM);
  const size_t lds = dec_gate_lds(d);
  hipError_t e = lds_attr(k_dec_gate<NW, IPW, MAXM, LOWRANK, MODE>, lds);
  if (e != hipSuccess) return e;
  ffn_launch((k_dec_gate<NW, IPW, MAXM, LOWRANK, MODE>), dim3(d.F / d.R), dim3(64 * NW), lds, s, d);
  return hipGetLastError();
}

template <int IPW, int MAXM, bool LOWRANK>
static hipError_t go_gate_mode(const DecodeDesc& d, hipStream_t s) {
  // 9..16 tokens: the split sequence only (also for a pack-only pass, up = 0)
  if constexpr (MAXM == 16) {
    if (d.up && d.mode != DEC_SPLIT) return hipErrorInvalidValue;
    return go_gate_k<IPW, MAXM, LOWRANK, DEC_SPLIT>(d, s);
  } else {
    // a pack-only pass (no hidden values) uses the chunk-mode kernel with up = 0
    const int mode = dec_gate_mode(d);
    if (mode == DEC_PART) return go_gate_k<IPW, MAXM, LOWRANK, DEC_PART>(d, s);
    if (mode == DEC_SPLIT) return go_gate_k<IPW, MAXM, LOWRANK, DEC_SPLIT>(d, s);
    return go_gate_k<IPW, MAXM, LOWRANK, DEC_CHUNK>(d, s);
  }
}

template <int IPW, int MAXM>
static hipError_t go_gate(const DecodeDesc& d, hipStream_t s) {
  return d.rank ? go_gate_mode<IPW, MAXM, true>(d, s) : go_gate_mode<IPW, MAXM, false>(d, s);
}

template <int MAXM>
static hipError_t go_gate_m(const DecodeDesc& d, hipStream_t s) {
  switch (d.ipw) {
    case 1: return go_gate<1, MAXM>(d, s);
    case 2: return go_gate<2, MAXM>(d, s);
    case 4: return go_gate<4, MAXM>(d, s);
    case 8:
      if constexpr (MAXM == 1) return go_gate<8, MAXM>(d, s);   // one token
      // several tokens: the low-rank gate over 64-row sub-tiles (on matrix
      // cores from 5 tokens)
      if (d.rank && d.K == 512 && d.R == 64) return go_gate_mode<8, MAXM, true>(d, s);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dec_gate(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM) return hipErrorInvalidValue;
  const int P = pow2_pieces(d.K);
  // 9..16 tokens with a full gate: 32-row sub-tiles on matrix cores
  const bool fg = d.M > 8 && !d.rank;
  if (fg ? (d.R != 32 || d.K % 128 != 0 || d.K > 128 * kFgMaxSteps || d.ipw != 4)
         : dec_gate_waves(dec_maxm(d.M)) * d.ipw != d.R * P)
    return hipErrorInvalidValue;
  if (d.R > 64 || d.R < 2 || d.T % d.R != 0 || d.F % d.R != 0 || d.T / d.R > 64) return hipErrorInvalidValue;
  switch (dec_maxm(d.M)) {
    case 1: return go_gate_m<1>(d, s);
    case 2: return go_gate_m<2>(d, s);
    case 4: return go_gate_m<4>(d, s);
    case 8: return go_gate_m<8>(d, s);
    default: return go_gate_m<16>(d, s);
  }
}

hipError_t launch_dec_reduce(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > 8 || d.d % 32 != 0 || d.F / d.R > kDecMaxSub || !d.part) return hipErrorInvalidValue;
  const dim3 grid(d.d / 32 + (d.route_pass ? 1 : 0)), blk(kRedThreads);
  switch (dec_maxm(d.M)) {
    case 1: ffn_launch((k_dec_reduce<1>), grid, blk, 0, s, d); break;
    case 2: ffn_launch((k_dec_reduce<2>), grid, blk, 0, s, d); break;
    case 4: ffn_launch((k_dec_reduce<4>), grid, blk, 0, s, d); break;
    default: ffn_launch((k_dec_reduce<8>), grid, blk, 0, s, d); break;
  }
  return hipGetLastError();
}

// Dynamic LDS of k_dec_up: x (M rows of d + 8 bf16; 16-byte multiple for d a
// multiple of 256), then the nsub sub-tile masks and prefixes.
size_t dec_up_lds(const DecodeDesc& d) { return (size_t)d.M * (d.d + 8) * 2 + (size_t)(d.F / d.R) * 12; }
// Static LDS of k_dec_up (s_scan, s_nrn, s_acc) and gfx950's LDS per workgroup.
constexpr size_t kUpStaticLds = kUpWaves * 4 + kUpNrnSlots * 4 + (size_t)kUpWaves * kUpNB * 64 * 16;
constexpr size_t kLdsPerWorkgroup = 160 * 1024;

// Sub-tile rows of the decode gate for m tokens, gate contraction K and
// TwELL tile T (0: the decode shape does not apply); *ipw gets the VALU
// pieces per wave. From 9 tokens a full gate uses 32-row sub-tiles on matrix
// cores.
int dec_gate_rows(int K, int T, int m, bool lowrank, int* ipw, int want_ipw) {
  // low rank, K = 512, 2..16 tokens (matrix cores from 5): 64-row sub-tiles
  // (8 pieces a wave) unless 4 pieces a wave (32 rows) are asked for
  if (lowrank && m >= 2 && m <= kDecMaxM && K == 512 && T % 64 == 0 && T / 64 <= 64 && want_ipw != 4) {
    if (ipw) *ipw = 8;
    return 64;
  }
  if (m > 8 && !lowrank) {
    if (K % 128 != 0 || K > 128 * kFgMaxSteps || T % 32 != 0 || T / 32 > 64) return 0;
    if (ipw) *ipw = 4;
    return 32;
  }
  return dec_rows_per_wg(K, T, m, ipw, want_ipw);
}

// Shapes the split sequence handles: d a multiple of 256 and at most 4096
// (a wave's eighth of d in registers), the tokens' x and the sub-tile masks
// within the up kernel's LDS (16 tokens at d = 4096), the padded list within
// the up grid's groups and each down workgroup's entries within its id buffer.
bool dec_split_ok(const DecodeDesc& d) {
  const int nkb = (d.F + 31) / 32;
  return d.d % 256 == 0 && d.d <= 32 * kUpWaves * kUpMaxSteps && (d.F + kUpGrid - 1) / kUpGrid <= kUpMaxEnt &&
         dec_up_lds(d) + kUpStaticLds + 512 <= kLdsPerWorkgroup &&
         d.F / d.R <= kDecMaxSub && d.ngroups >= 1 && d.ngroups <= 32 && (nkb + d.ngroups - 1) / d.ngroups * 32 <= kDown2MaxIds &&
         d.ldh >= nkb * 32;
}

hipError_t launch_dec_up(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || !dec_split_ok(d) || !d.ad || !d.ul_nrn || !d.ul_h || !d.ul_total)
    return hipErrorInvalidValue;
  const size_t lds = dec_up_lds(d);
  hipError_t e = lds_attr(k_dec_up, lds);
  if (e != hipSuccess) return e;
  ffn_launch(k_dec_up, dim3(kUpGrid), dim3(64 * kUpWaves), lds, s, d);
  return hipGetLastError();
}

// Entry groups of the split down kernel: about 512 workgroups in all, and
// enough groups that each holds at most kDown2MaxIds list entries.
int dec_down2_groups(int d_model, int d_ff) {
  const int nsl = std::max(1, d_model / 64), nkb = (d_ff + 31) / 32;
  const int need = (nkb * 32 + kDown2MaxIds - 1) / kDown2MaxIds;
  return std::max(need, std::max(1, std::min(32, 512 / nsl)));
}

hipError_t launch_dec_down2(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || d.d % 64 != 0 || !dec_split_ok(d) || !d.ul_nrn || !d.ul_h || !d.ul_total ||
      !d.part)
    return hipErrorInvalidValue;
  ffn_launch(k_dec_down2, dim3(d.d / 64 * d.ngroups), dim3(kDown2Threads), 0, s, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = d.M * d.d;
  ffn_launch(k_dec_reduce2, dim3((n + 1023) / 1024 + (d.route_pass ? 1 : 0)), dim3(256), 0, s, d);
  return hipGetLastError();
}

int dec_rows_per_wg(int K, int T, int m, int* ipw_out, int want_ipw) {
  const int P = pow2_pieces(K);
  if (P > 8 || m < 1 || m > kDecMaxM) return 0;
  const int nw = dec_gate_waves(dec_maxm(m));
  // pieces per wave: by default 8 for one token (more of each wave's loads in
  // flight, fewer workgroups and partial rows; 1B decode gate 16.7 -> 13.1 us)
  // and 4 otherwise, down to 1 until the rows fit; `want_ipw` (8 for one token
  // only) is tried first
  const int first = (want_ipw == 8 && m == 1) || want_ipw == 4 || want_ipw == 2 || want_ipw == 1 ? want_ipw
                                                                                            : (m == 1 ? 8 : 4);
  for (int ipw = first; ipw >= 1; ipw >>= 1) {
    const int R = nw * ipw / P;
    if (R >= 2 && R <= 64 && T % R == 0 && T / R <= 64) {
      if (ipw_out) *ipw_out = ipw;
      return R;
    }
  }
  return 0;
}

hipError_t launch_dec_down(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > 8 || d.d % 64 != 0 || d.F / d.R > kDecMaxSub) return hipErrorInvalidValue;
  const dim3 grid(d.d / 8 + (d.route_pass ? 1 : 0)), blk(kDownThreads);
  switch (dec_maxm(d.M)) {
    case 1: ffn_launch((k_dec_down<1>), grid, blk, 0, s, d); break;
    case 2: ffn_launch((k_dec_down<2>), grid, blk, 0, s, d); break;
    case 4: ffn_launch((k_dec_down<4>), grid, blk, 0, s, d); break;
    default: ffn_launch((k_dec_down<8>), grid, blk, 0, s, d); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ grouped one-token launches
// One launch of each one-token kernel for several FFNs of one shape (a
// mixture-of-experts layer's active experts): grid.y picks the FFN's
// descriptor, so each expert's workgroups run exactly its own kernel's work.
hipError_t launch_dec_lowrank_group(const DecGroup& g, int n, hipStream_t s) {
  const DecodeDesc& d = g.d[0];
  if (n < 1 || n > kDecGroupMax || d.M != 1 || d.rank <= 0 || d.nslab > 0) return hipErrorInvalidValue;
  const int P = pow2_pieces(d.d);
  if (P > 8) return hipErrorInvalidValue;
  DecGroup gl = g;                                   // ipw carries the pieces per V row here
  for (int i = 0; i < n; ++i) gl.d[i].ipw = P;
  auto go = [&](auto kern, int IPW) -> hipError_t {
    const int R = kDecVWaves * IPW / P;
    const size_t lds = dec_lowrank_lds(d);
    hipError_t e = lds_attr(kern, lds);
    if (e != hipSuccess) return e;
    ffn_launch(kern, dim3((d.rank + R - 1) / R, n), dim3(64 * kDecVWaves), lds, s, gl);
    return hipGetLastError();
  };
  if (P >= 8) return go(k_dec_lowrank_grp<4, 1>, 4);
  return go(k_dec_lowrank_grp<2, 1>, 2);
}

hipError_t launch_dec_gate_group(const DecGroup& g, int n, hipStream_t s) {
  const DecodeDesc& d = g.d[0];
  if (n < 1 || n > kDecGroupMax || d.M != 1 || d.mode != DEC_PART || !d.up) return hipErrorInvalidValue;
  constexpr int NW = dec_gate_waves(1);
  const int P = pow2_pieces(d.K);
  if (NW * d.ipw != d.R * P || d.R > 64 || d.R < 2 || d.T % d.R != 0 || d.F % d.R != 0 || d.T / d.R > 64)
    return hipErrorInvalidValue;
  const size_t lds = dec_gate_lds(d);
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = lds_attr(kern, lds);
    if (e != hipSuccess) return e;
    ffn_launch(kern, dim3(d.F / d.R, n), dim3(64 * NW), lds, s, g);
    return hipGetLastError();
  };
  const bool lr = d.rank > 0;
  switch (d.ipw) {
    case 1: return lr ? go(k_dec_gate_grp<NW, 1, 1, true, DEC_PART>) : go(k_dec_gate_grp<NW, 1, 1, false, DEC_PART>);
    case 2: return lr ? go(k_dec_gate_grp<NW, 2, 1, true, DEC_PART>) : go(k_dec_gate_grp<NW, 2, 1, false, DEC_PART>);
    case 4: return lr ? go(k_dec_gate_grp<NW, 4, 1, true, DEC_PART>) : go(k_dec_gate_grp<NW, 4, 1, false, DEC_PART>);
    case 8: return lr ? go(k_dec_gate_grp<NW, 8, 1, true, DEC_PART>) : go(k_dec_gate_grp<NW, 8, 1, false, DEC_PART>);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dec_reduce_group(const DecGroup& g, int n, hipStream_t s) {
  const DecodeDesc& d = g.d[0];
  if (n < 1 || n > kDecGroupMax || d.M != 1 || d.d % 32 != 0 || d.F / d.R > kDecMaxSub || !d.part)
    return hipErrorInvalidValue;
  ffn_launch(k_dec_reduce_grp<1>, dim3(d.d / 32 + (d.route_pass ? 1 : 0), n), dim3(kRedThreads), 0, s, g);
  return hipGetLastError();
}

// ------------------------------------------------------------------ grouped split-sequence launches
// The same for FFNs of one shape with 2..8 tokens each, planned for the
// group's largest token count (so every descriptor shares the launch shape:
// sub-tile rows, pieces, slabs, entry groups) and each carrying its own count.
// Whether a split-sequence plan has the one shape the grouped gate is built
// for (low rank 512, 64-row sub-tiles of 8 pieces) and the other stages fit.
bool dec_split_group_shape(const DecodeDesc& d) {
  return d.rank > 0 && d.K == 512 && d.ipw == 8 && d.R == 64 && d.nslab > 0 && d.rank % 16 == 0 &&
         lowrank_mf_waves(d.d, d.nslab) != 0 && d.d % 64 == 0 && d.T % d.R == 0 && d.F % d.R == 0 &&
         d.T / d.R <= 64 && dec_split_ok(d);
}

static bool split_group_ok(const DecGroup& g, int n) {
  if (n < 1 || n > kDecGroupMax) return false;
  const DecodeDesc& a = g.d[0];
  for (int i = 0; i < n; ++i) {
    const DecodeDesc& b = g.d[i];
    if (b.M < 2 || b.M > 8 || b.mode != DEC_SPLIT || !b.up || b.d != a.d || b.F != a.F || b.T != a.T ||
        b.K != a.K || b.rank != a.rank || b.R != a.R || b.ipw != a.ipw || b.nslab != a.nslab ||
        b.ngroups != a.ngroups || b.ldh != a.ldh || !dec_split_ok(b))
      return false;
  }
  return dec_split_group_shape(a);
}
static int group_maxm_of(const DecGroup& g, int n) {
  int mx = 1;
  for (int i = 0; i < n; ++i) mx = std::max(mx, g.d[i].M);
  return dec_maxm(mx);
}

hipError_t launch_dec_split_group(const DecGroup& g, int n, int stage, hipStream_t s) {
  if (!split_group_ok(g, n)) return hipErrorInvalidValue;
  const DecodeDesc& d = g.d[0];
  const int maxm = group_maxm_of(g, n);
  if (stage == 0) {                                    // t = V x on matrix cores, nslab slabs each
    const int nwv = lowrank_mf_waves(d.d, d.nslab);
    if (nwv == 0 || d.rank % 16 != 0) return hipErrorInvalidValue;
    ffn_launch(k_dec_lowrank_mf_grp, dim3(d.rank / 16, d.nslab, n), dim3(64 * nwv), 0, s, g);
    return hipGetLastError();
  }
  if (stage == 1) {                                    // gate, selection, pack, union activations
    if (d.ipw != 8 || d.K != 512 || d.R != 64 || d.T % d.R != 0 || d.F % d.R != 0 || d.T / d.R > 64)
      return hipErrorInvalidValue;
    size_t lds = 0;
    for (int i = 0; i < n; ++i) {
      DecodeDesc t = g.d[i];
      t.M = maxm;
      lds = std::max(lds, dec_gate_lds(t));
    }
    auto go = [&](auto kern) -> hipError_t {
      hipError_t e = lds_attr(kern, lds);
      if (e != hipSuccess) return e;
      ffn_launch(kern, dim3(d.F / d.R, n), dim3(64 * dec_gate_waves(maxm)), lds, s, g);
      return hipGetLastError();
    };
    switch (maxm) {
      case 2: return go(k_dec_gate_grp<dec_gate_waves(2), 8, 2, true, DEC_SPLIT>);
      case 4: return go(k_dec_gate_grp<dec_gate_waves(4), 8, 4, true, DEC_SPLIT>);
      case 8: return go(k_dec_gate_grp<dec_gate_waves(8), 8, 8, true, DEC_SPLIT>);
    }
    return hipErrorInvalidValue;
  }
  if (stage == 2) {                                    // up products of the union list
    size_t lds = 0;
    for (int i = 0; i < n; ++i) lds = std::max(lds, dec_up_lds(g.d[i]));
    hipError_t e = lds_attr(k_dec_up_grp, lds);
    if (e != hipSuccess) return e;
    ffn_launch(k_dec_up_grp, dim3(kUpGrid, n), dim3(64 * kUpWaves), lds, s, g);
    return hipGetLastError();
  }
  if (stage == 3) {                                    // down products, then the ordered group sum
    if (d.d % 64 != 0) return hipErrorInvalidValue;
    ffn_launch(k_dec_down2_grp, dim3(d.d / 64 * d.ngroups, n), dim3(kDown2Threads), 0, s, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nmax = 0;
    for (int i = 0; i < n; ++i) nmax = std::max(nmax, g.d[i].M * g.d[i].d);
    ffn_launch(k_dec_reduce2_grp, dim3((nmax + 1023) / 1024 + 1, n), dim3(256), 0, s, g);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace ffn
