// Skinny GEMM for 9..64 tokens per workgroup on gfx950: C[n, m] = sum_k
// A[n, k] B[m, k] with many weight rows n (the FFN's products at a few dozen
// tokens are weight streams: about 2 * 64 FLOP per weight byte at 64 tokens,
// far below the matrix cores' ratio, so the bound is HBM).
//
// A workgroup of four waves owns 64 weight rows and every token of its
// 16 * MB-token block, so the L2 reads of the token operand stay within the
// weight bytes. The K loop runs in steps of KS elements: the step's token
// tile (16 MB rows x KS, bf16; for an fp32 B its bf16 hi and lo parts) is
// staged once in LDS (two stages, one barrier a step) and shared by the four
// waves. A wave multiplies its RB 16-row blocks with its share of the step's
// chunks on v_mfma_f32_16x16x32_bf16; its weight loads go straight from HBM
// into registers in the MFMA operand layout, two steps ahead, so the stream
// does not wait for the arithmetic. A token tile is loaded two steps ahead
// too, so waiting for it never waits for weight loads still in flight (the
// wait counter completes loads in issue order). Partial tiles of
// waves that split a step are added in LDS in wave order, and the fp32 tile
// goes through the same epilogues as the other GEMM kernels.
//
// The down projection (d_model rows, d_ff long) has too few 64-row tiles for
// the chip, so its K range is split over ks workgroups (blockIdx.z); each
// writes an fp32 partial slab and k_sk_ksum adds the slabs in slice order.
#include <algorithm>

#include "gemm_core.cuh"

namespace ffn {

constexpr int kSkThreads = 256;  // four waves
constexpr int kSkNT = 64;        // weight rows per workgroup
constexpr int kSkPad = 8;        // bf16 padding of an LDS token row: rows start 4 banks apart

template <int BM>
struct SkStep {
  static constexpr bool SPLIT = BM == B_F32_SPLIT;
  static constexpr int KS = SPLIT ? 128 : 256;      // K elements per step
  static constexpr int C = KS / 32;                 // MFMA chunks per step
  static constexpr int NB = SPLIT ? 2 : 1;          // LDS token tiles per stage (hi, lo)
  static constexpr int LDB = KS + kSkPad;           // bf16 per LDS token row
  static constexpr int ESZ = SPLIT ? 4 : 2;         // bytes per global B element
};

// Wave layout of a 64-row tile: WN waves along the rows, each RB 16-row
// blocks, and WK = 4 / WN waves splitting every step's chunks. At 64 tokens
// a wave takes 32 rows (RB = 2), which halves the LDS token reads per weight
// byte; otherwise 16 rows and the whole step.
template <int MB>
struct SkWaves {
  static constexpr int RB = MB == 4 ? 2 : 1;
  static constexpr int WN = 4 / RB;
  static constexpr int WK = 4 / WN;
};

template <int MB, int BM>
constexpr size_t sk_lds_bytes() {
  using S = SkStep<BM>;
  const size_t b = (size_t)2 * S::NB * 16 * MB * S::LDB * 2;   // two stages
  const size_t t = (size_t)kSkNT * (16 * MB + 1) * 4;
  return b > t ? b : t;
}

template <int MB, int BM, int NMAT, int EPI>
__global__ __launch_bounds__(kSkThreads) void k_gemm_sk(const GemmDesc g, const EpiDesc e) {
  using S = SkStep<BM>;
  using W = SkWaves<MB>;
  constexpr int RB = W::RB, WN = W::WN, WK = W::WK;
  constexpr int NT = kSkNT, MT = 16 * MB, LDT = MT + 1, RPM = NT / NMAT;
  constexpr int CPW = S::C / WK;                    // chunks of a step per wave
  constexpr int RS = 2;                             // steps of weight chunks in flight
  constexpr int RING = RS * RB * CPW;
  constexpr int CPR = S::KS * S::ESZ / 16;          // 16-byte global pieces per token row and step
  constexpr int BPT = MT * CPR / kSkThreads;        // token-tile pieces per thread and step
  constexpr int STAGE = S::NB * MT * S::LDB;        // bf16 per LDS stage
  static_assert(16 * RB * WN == NT && S::C % WK == 0 && (MT * CPR) % kSkThreads == 0, "tile shape");
  extern __shared__ uint4 s_dyn[];
  uint16_t* s_b = reinterpret_cast<uint16_t*>(s_dyn);   // two stages [NB][MT][LDB] during the K loop
  float* tile = reinterpret_cast<float*>(s_dyn);         // [NT][LDT] afterwards

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int tile_id = blockIdx.x, m0 = blockIdx.y * MT;
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  if (m0 >= Mtot) return;                           // uniform over the workgroup
  const int mcnt = min(MT, Mtot - m0);
  const int n0 = tile_id * RPM;
  // this workgroup's K steps (the host checks K % KS == 0 and ks <= steps)
  const int ks = gridDim.z, z = blockIdx.z, steps_all = g.K / S::KS;
  const int st0 = z * steps_all / ks, nsteps = (z + 1) * steps_all / ks - st0;
  // the workgroups start their step sequences at different steps (wrapping
  // around), so the loads in flight across the chip spread over the rows'
  // whole length rather than one column range of rows a fixed stride apart
  const int rot = (int)(((unsigned)tile_id * 5u + (unsigned)blockIdx.y) % (unsigned)nsteps);
  auto mstep = [&](int s) { return s + rot < nsteps ? s + rot : s + rot - nsteps; };

  // this lane's weight rows (operand lane l: row l % 16 of block rb, 8
  // elements at (l / 16) * 8)
  const uint16_t* ap[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (wn * RB + rb) * 16 + (lane & 15);
    ap[rb] = reinterpret_cast<const uint16_t*>(r / RPM ? g.A1 : g.A0) + (size_t)(n0 + r % RPM) * g.lda +
             (size_t)st0 * S::KS + (lane >> 4) * 8 + wk * CPW * 32;
  }

  // token tile pieces of this thread: row p / CPR, 16-byte piece p % CPR
  const char* bsrc[BPT];
  bool bok[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int p = threadIdx.x + i * kSkThreads, row = p / CPR, c = p % CPR;
    bok[i] = row < mcnt;
    const int brow = bok[i] ? (g.gather ? g.gather[m0 + row] : m0 + row) : 0;
    bsrc[i] = reinterpret_cast<const char*>(g.B) + ((size_t)brow * g.ldb + (size_t)st0 * S::KS) * S::ESZ + (size_t)c * 16;
  }
  // two register buffers of token pieces: the tile of step s + 2 is loaded
  // at the start of step s, and the tile of step s + 1 (loaded a step
  // earlier) is stored to LDS at its end
  uint4 rbuf[2][BPT];
  auto load_b = [&](uint4 (&rb_)[BPT], int s) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) rb_[i] = bok[i] ? ldg16(bsrc[i] + (size_t)mstep(s) * S::KS * S::ESZ) : uint4{0, 0, 0, 0};
  };
  auto store_b = [&](const uint4 (&rb_)[BPT], int stage) {
    uint16_t* dst = s_b + (size_t)stage * STAGE;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int p = threadIdx.x + i * kSkThreads, row = p / CPR, c = p % CPR;
      if constexpr (S::SPLIT) {
        // four fp32 values -> bf16 hi = bf16(t), lo = bf16(t - hi)
        const float x[4] = {__uint_as_float(rb_[i].x), __uint_as_float(rb_[i].y), __uint_as_float(rb_[i].z),
                            __uint_as_float(rb_[i].w)};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hi[q] = f2bf(x[q]);
          lo[q] = f2bf(x[q] - bf2f(hi[q]));
        }
        *reinterpret_cast<uint2*>(dst + (size_t)row * S::LDB + c * 4) = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
        *reinterpret_cast<uint2*>(dst + (size_t)(MT + row) * S::LDB + c * 4) =
            uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      } else {
        *reinterpret_cast<uint4*>(dst + (size_t)row * S::LDB + c * 8) = rb_[i];
      }
    }
  };

  // weight ring: block rb, chunk j of step s sits in slot ((s % RS) * RB + rb)
  // * CPW + j; a load past the last step re-reads the last step (never used).
  // Loads complete in issue order for the wait counter, and the token tile
  // stored at the end of step s was issued at the start of step s - 1, ahead
  // of the weight refills of steps s - 1 and s: those stay in flight.
  uint4 ra[RING];
#pragma unroll
  for (int q = 0; q < RS; ++q)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        ra[(q * RB + rb) * CPW + j] = ldg16(ap[rb] + (size_t)mstep(min(q, nsteps - 1)) * S::KS + j * 32);
  load_b(rbuf[0], 0);
  store_b(rbuf[0], 0);
  if (nsteps > 1) load_b(rbuf[1], 1);
  __syncthreads();

  f32x4_t acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // LDS offset of this lane's token operand: token 16 mb + l % 16, element
  // (wk * CPW + j) * 32 + (l / 16) * 8 of the step
  const int boff = (lane & 15) * S::LDB + wk * CPW * 32 + (lane >> 4) * 8;

  for (int s0 = 0; s0 < nsteps; s0 += RS) {
#pragma unroll
    for (int q = 0; q < RS; ++q) {
      const int s = s0 + q;
      if (s < nsteps) {                             // uniform
        if (s + 2 < nsteps) load_b(rbuf[q], s + 2);  // rbuf[s % 2] was stored at the end of step s - 1
        const uint16_t* bl = s_b + (size_t)q * STAGE + boff;   // stage s % 2 (RS = 2)
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          uint4 bf[MB][S::NB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < S::NB; ++nb)
              bf[mb][nb] = *reinterpret_cast<const uint4*>(bl + (size_t)(nb * MT + mb * 16) * S::LDB + j * 32);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int slot = (q * RB + rb) * CPW + j;
            const uint4 a = ra[slot];
            ra[slot] = ldg16(ap[rb] + (size_t)mstep(min(s + RS, nsteps - 1)) * S::KS + j * 32);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int nb = 0; nb < S::NB; ++nb)
                acc[rb][mb] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bf[mb][nb]), acc[rb][mb], 0, 0, 0);
          }
        }
        // the other stage was last read in the previous step, which every
        // wave finished before the previous barrier
        if (s + 1 < nsteps) store_b(rbuf[(q + 1) & 1], (q + 1) & 1);
        __syncthreads();
      }
    }
  }

  // fixed-order sum of the WK partial tiles (the LDS tokens are no longer read)
  for (int w = 0; w < WK; ++w) {
    if (wk == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            float* p = &tile[((wn * RB + rb) * 16 + 4 * (lane >> 4) + vv) * LDT + mb * 16 + (lane & 15)];
            if (w == 0) *p = acc[rb][mb][vv];
            else *p += acc[rb][mb][vv];
          }
    }
    __syncthreads();
  }
  if (ks > 1) {
    // a K slice: the fp32 partial slab, summed in order by k_sk_ksum
    if constexpr (EPI == EPI_Y) {
      float* out = g.skpart + (size_t)z * g.M * g.nrows;
      for (int p = threadIdx.x; p < NT * mcnt; p += kSkThreads) {
        const int rr = p % NT, m = p / NT;
        out[(size_t)(m0 + m) * g.nrows + n0 + rr] = tile[rr * LDT + m];
      }
    }
    return;
  }
  if (EPI == EPI_TWELL && BM == B_F32_SPLIT && e.t_out && tile_id == 0) store_summed_t(g, e, m0, mcnt);
  const TileView v{tile, LDT, NT, n0, m0, mcnt, RPM};
  run_epilogue<NMAT, EPI>(e, v, g.ctrl, 0);
}

// y rows of a K-split product: the ks partial slabs added in slice order, for
// the first min(M, m_dev) token slots (output row yrows[m]).
__global__ __launch_bounds__(256) void k_sk_ksum(const GemmDesc g, const EpiDesc e, int ks) {
  int Mtot = g.M;
  if (g.m_dev) Mtot = min(Mtot, *g.m_dev);
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= g.nrows) return;
  for (int m = blockIdx.y; m < Mtot; m += gridDim.y) {
    float4 acc = *reinterpret_cast<const float4*>(g.skpart + (size_t)m * g.nrows + n);
    for (int z = 1; z < ks; ++z) {
      const float4 p = *reinterpret_cast<const float4*>(g.skpart + ((size_t)z * g.M + m) * g.nrows + n);
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

// ------------------------------------------------------------------ dispatch
// Tile shape of the skinny kernel: 64 weight rows per workgroup (the L2 reads
// of the token tile then stay within the weight bytes) and ks K slices. Output
// rows (the down projection: d_model rows, d_ff long) split K up to 8 ways,
// each slice at least two steps, until the tiles fill the CUs, when the
// partial buffer holds the slabs. A TwELL gate needs the 32 or 64 rows of a
// matrix to divide the TwELL tile. Returns false when the shape does not apply.
static bool sk_shape(const GemmDesc& g, const EpiDesc& e, int cus, int* ks_out) {
  if (g.dtype != DT_BF16 || g.gemv || g.ks != 1 || g.M < 1) return false;
  if (g.mt != 16 && g.mt != 32 && g.mt != 64) return false;
  int ksz = 0;
  if (g.bmode == B_NATIVE && g.b_nsum == 1) ksz = SkStep<B_NATIVE>::KS;
  if (g.bmode == B_F32_SPLIT && g.b_nsum == 1) ksz = SkStep<B_F32_SPLIT>::KS;
  if (ksz == 0 || g.K % ksz != 0) return false;
  const int rpm = kSkNT / g.nmat;
  if (g.nrows % rpm != 0 || (e.kind == EPI_TWELL && e.T % rpm != 0)) return false;
  const int steps = g.K / ksz;
  const int tiles = g.nrows / rpm * ((g.M + g.mt - 1) / g.mt);
  int ks = 1;
  if (e.kind == EPI_Y && g.nmat == 1 && g.skpart && g.nrows % 4 == 0) {
    while (tiles * ks < cus && ks < 8 && steps / (2 * ks) >= 2 && (size_t)(2 * ks) * g.M <= (size_t)g.skpart_rows)
      ks *= 2;
  }
  // too few tiles for the chip without a K split: the per-wave kernels
  if (tiles * ks < cus / 2) return false;
  *ks_out = ks;
  return true;
}

bool sk_ok(const GemmDesc& g, const EpiDesc& e) {
  int ks;
  return sk_shape(g, e, 256, &ks);
}

template <int MB, int BM, int NMAT, int EPI>
static hipError_t go_sk(const GemmDesc& g, const EpiDesc& e, int ks, hipStream_t s) {
  constexpr size_t lds = sk_lds_bytes<MB, BM>();
  auto kern = k_gemm_sk<MB, BM, NMAT, EPI>;
  if (lds > 64 * 1024) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  const dim3 grid(g.nrows * g.nmat / kSkNT, (g.M + g.mt - 1) / g.mt, ks);
  ffn_launch(kern, grid, dim3(kSkThreads), lds, s, g, e);
  return hipGetLastError();
}

template <int BM, int NMAT, int EPI>
static hipError_t sk_mb(const GemmDesc& g, const EpiDesc& e, int ks, hipStream_t s) {
  switch (g.mt) {
    case 16: return go_sk<1, BM, NMAT, EPI>(g, e, ks, s);
    case 32: return go_sk<2, BM, NMAT, EPI>(g, e, ks, s);
    case 64: return go_sk<4, BM, NMAT, EPI>(g, e, ks, s);
  }
  return hipErrorInvalidValue;
}

static hipError_t sk_epi(const GemmDesc& g, const EpiDesc& e, int ks, hipStream_t s) {
  if (g.bmode == B_F32_SPLIT) {
    switch (e.kind) {
      case EPI_STORE_F32: return sk_mb<B_F32_SPLIT, 1, EPI_STORE_F32>(g, e, ks, s);
      case EPI_TWELL: return sk_mb<B_F32_SPLIT, 1, EPI_TWELL>(g, e, ks, s);
    }
    return hipErrorInvalidValue;
  }
  switch (e.kind) {
    case EPI_STORE_F32: return sk_mb<B_NATIVE, 1, EPI_STORE_F32>(g, e, ks, s);
    case EPI_TWELL: return sk_mb<B_NATIVE, 1, EPI_TWELL>(g, e, ks, s);
    case EPI_WINA: return g.nmat == 2 ? sk_mb<B_NATIVE, 2, EPI_WINA>(g, e, ks, s) : hipErrorInvalidValue;
    case EPI_DENSE_H:
      return g.nmat == 2 ? sk_mb<B_NATIVE, 2, EPI_DENSE_H>(g, e, ks, s) : sk_mb<B_NATIVE, 1, EPI_DENSE_H>(g, e, ks, s);
    case EPI_Y: return g.nmat == 1 ? sk_mb<B_NATIVE, 1, EPI_Y>(g, e, ks, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_sk(const GemmDesc& g, const EpiDesc& e, hipStream_t s) {
  GemmDesc q = g;
  int ks = 1;
  if (!sk_shape(g, e, 256, &ks)) return hipErrorInvalidValue;
  q.nt = kSkNT;
  hipError_t err = sk_epi(q, e, ks, s);
  if (err != hipSuccess || ks == 1) return err;
  ffn_launch(k_sk_ksum, dim3((q.nrows / 4 + 255) / 256, std::min(q.M, 64)), dim3(256), 0, s, q, e, ks);
  return hipGetLastError();
}

}  // namespace ffn
