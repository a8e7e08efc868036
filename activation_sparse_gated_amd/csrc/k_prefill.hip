// Prefill-shaped GEMM of the sparse gated FFN on gfx950 matrix cores.
//
// C[n, m] = sum_k A[n, k] B[m, k] for many tokens (M >= 128): A holds weight
// rows (one matrix, or the gate and up rows of the same neurons stacked per
// tile), B token rows, both K-contiguous bf16. A workgroup of 4 waves owns a
// 128 (weight rows) x 128 (tokens) tile and walks K in steps of 64 with two LDS
// stages: the next step's 32 KB is loaded into registers (16-byte loads, 8
// threads per 128-byte row segment) while the current step is multiplied from
// LDS, then stored to the other stage. Each wave computes a 64 x 64 quadrant
// with v_mfma_f32_16x16x32_bf16 (operand lane l: row l % 16, k (l / 16) * 8;
// accumulator lane l: row 4 (l / 16) + v, column l % 16). LDS rows are 8
// chunks of 16 bytes stored at chunk c ^ (row % 8), so the 16 rows one MFMA
// operand read touches fall in distinct banks.
//
// The fp32 result tile (128 x 128, padded rows) is written to LDS, reusing the
// staging buffers, and handed to the same epilogues as the decode-shaped
// kernels (gemm_core.cuh) in one pass: activation,
// selection and TwELL pack for the gate [Sparser/Faster/Lighter page,
// "TwELL 減掉轉換開銷"], dense hidden values, output rows, WINA scores.
#include "gemm_core.cuh"

namespace ffn {

constexpr int PF_BN = 128, PF_BM = 128, PF_BK = 64, PF_THREADS = 256;

__device__ __forceinline__ int pf_slot(int row, int c) { return row * 8 + (c ^ (row & 7)); }

template <int NMAT, int EPI>
__global__ __launch_bounds__(PF_THREADS) void k_gemm_pf(const GemmDesc g, const EpiDesc e) {
  constexpr int RPM = PF_BN / NMAT;
  constexpr int LDT = PF_BM + 1;                        // C tile: 128 rows x 128 tokens (+1 pad)
  // 2 stages x (A, B) x 128 rows x 8 chunks = 64 KB for the K loop, then the
  // fp32 C tile (66 KB) for the epilogue
  constexpr int SMEM16 = (PF_BN * LDT * 4 + 15) / 16 > 2 * 2 * PF_BN * 8 ? (PF_BN * LDT * 4 + 15) / 16 : 2 * 2 * PF_BN * 8;
  __shared__ uint4 smem[SMEM16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int tile_id = blockIdx.x, n0 = tile_id * RPM;
  const int m0 = blockIdx.y * PF_BM;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;
  const int mcnt = min(PF_BM, Mtot - m0);

  // per-thread global sources: 4 A chunks and 4 B chunks per K step
  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
  int arow[4], ach[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + PF_THREADS * i, r = q >> 3, c = q & 7;
    arow[i] = r;
    ach[i] = c;
    const int mat = r / RPM, rr = n0 + (r % RPM);
    asrc[i] = reinterpret_cast<const uint16_t*>(mat ? g.A1 : g.A0) + (size_t)rr * g.lda + c * 8;
    const int tok = m0 + r;
    bsrc[i] = nullptr;
    if (r < mcnt) {
      const int brow = g.gather ? g.gather[tok] : tok;
      bsrc[i] = reinterpret_cast<const uint16_t*>(g.B) + (size_t)brow * g.ldb + c * 8;
    }
  }
  uint4 ra[4], rb[4];
  auto fetch = [&](int kt) {
    const size_t ko = (size_t)kt * PF_BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ldg16(asrc[i] + ko);
      rb[i] = bsrc[i] ? ldg16(bsrc[i] + ko) : uint4{0, 0, 0, 0};
    }
  };
  auto stash = [&](int st) {
    uint4* sa = smem + st * (2 * PF_BN * 8);
    uint4* sb = sa + PF_BN * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[pf_slot(arow[i], ach[i])] = ra[i];
      sb[pf_slot(arow[i], ach[i])] = rb[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K steps of this workgroup: all of them, or slice blockIdx.z of g.ks
  const int KTA = g.K / PF_BK;
  const int kt0 = (int)((long long)KTA * blockIdx.z / g.ks), KT = (int)((long long)KTA * (blockIdx.z + 1) / g.ks);
  fetch(kt0);
  stash(0);
  __syncthreads();
  for (int kt = kt0; kt < KT; ++kt) {
    const int st = (kt - kt0) & 1;
    if (kt + 1 < KT) fetch(kt + 1);
    const uint4* sa = smem + st * (2 * PF_BN * 8);
    const uint4* sb = sa + PF_BN * 8;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      uint4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = sa[pf_slot(wn * 64 + i * 16 + (lane & 15), c)];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = sb[pf_slot(wm * 64 + j * 16 + (lane & 15), c)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) stash(st ^ 1);
    __syncthreads();
  }

  if (g.ks > 1) {
    // split K: this slice's fp32 partial tile, four consecutive rows a lane
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = wm * 64 + j * 16 + (lane & 15), r = wn * 64 + i * 16 + 4 * (lane >> 4);
        if (m < mcnt)
          *reinterpret_cast<float4*>(g.kpart + ((size_t)blockIdx.z * g.kpart_m + m0 + m) * g.nrows + n0 + r) =
              float4{acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      }
    return;
  }

  // epilogue on the whole 128 x 128 tile through fp32 LDS: one pass (one
  // look-back round for the TwELL pack) per workgroup
  float* tile = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        tile[(wn * 64 + i * 16 + 4 * (lane >> 4) + v) * LDT + wm * 64 + j * 16 + (lane & 15)] = acc[i][j][v];
  __syncthreads();
  const TileView tv{tile, LDT, PF_BN, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(e, tv, g.ctrl, 0);
}

// Whether the prefill kernel handles this GEMM (host side).
bool pf_ok(const GemmDesc& g, const EpiDesc& e) {
  if (g.dtype != DT_BF16 || g.bmode != B_NATIVE || g.b_nsum != 1 || g.gemv) return false;
  if (g.ks != 1 && (g.ks < 1 || g.nmat != 1 || e.kind != EPI_Y || !g.kpart || !g.m_dev || g.kpart_m < g.M ||
                    g.K / PF_BK < g.ks))
    return false;
  if (g.M < PF_BM || g.K % PF_BK != 0 || (g.nrows * g.nmat) % PF_BN != 0) return false;
  if (g.nmat == 2 && g.nrows % (PF_BN / 2) != 0) return false;
  if (e.kind == EPI_TWELL && (e.T % PF_BN != 0 || e.t_out)) return false;
  if (e.kind == EPI_STORE_F32) return false;
  return true;
}

template <int NMAT, int EPI>
static hipError_t go_pf(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  const dim3 grid(g.nrows * g.nmat / PF_BN, (g.M + PF_BM - 1) / PF_BM, g.ks);
  ffn_launch((k_gemm_pf<NMAT, EPI>), grid, dim3(PF_THREADS), 0, s, g, e);
  return hipGetLastError();
}

// y rows of a split-K product: the sum of the g.ks partial slices in slice
// order, for the first m_dev token slots (output row yrows[m]).
__global__ __launch_bounds__(256) void k_pf_ksum(const GemmDesc g, const EpiDesc e) {
  const int Mtot = min(g.M, *g.m_dev);
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= g.nrows) return;
  for (int m = blockIdx.y; m < Mtot; m += gridDim.y) {
    float4 acc = float4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < g.ks; ++z) {
      const float4 p = *reinterpret_cast<const float4*>(g.kpart + ((size_t)z * g.kpart_m + m) * g.nrows + n);
      acc.x += p.x;
      acc.y += p.y;
      acc.z += p.z;
      acc.w += p.w;
    }
    const size_t row = (size_t)(e.yrows ? e.yrows[m] : m) * e.ldy + n;
    if (e.out_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(e.y) + row) = acc;
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(e.y) + row) =
          uint2{f2bf(acc.x) | (f2bf(acc.y) << 16), f2bf(acc.z) | (f2bf(acc.w) << 16)};
    }
  }
}

hipError_t launch_pf_ksum(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  if (g.ks <= 1 || !g.kpart || !g.m_dev || g.nrows % 4 != 0) return hipErrorInvalidValue;
  ffn_launch(k_pf_ksum, dim3((g.nrows / 4 + 255) / 256, 256), dim3(256), 0, s, g, e);
  return hipGetLastError();
}

hipError_t launch_gemm_pf(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  switch (e.kind) {
    case EPI_TWELL: return g.nmat == 1 ? go_pf<1, EPI_TWELL>(g, e, s) : hipErrorInvalidValue;
    case EPI_DENSE_H: return g.nmat == 2 ? go_pf<2, EPI_DENSE_H>(g, e, s) : go_pf<1, EPI_DENSE_H>(g, e, s);
    case EPI_Y: return g.nmat == 1 ? go_pf<1, EPI_Y>(g, e, s) : hipErrorInvalidValue;
    case EPI_WINA: return g.nmat == 2 ? go_pf<2, EPI_WINA>(g, e, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace ffn
