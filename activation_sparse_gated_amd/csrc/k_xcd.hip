// Sparse up and down products over the TwELL pack at prefill token counts,
// organised around the eight XCDs' separate L2 caches.
//
// At thousands of tokens every weight row is gathered by many tokens, so the
// per-token sparse kernel re-reads W_up and W_down from the last-level cache
// about (active entries x 2 rows) times. Workgroups are dealt to the eight XCDs
// round-robin (workgroup b runs on XCD b % 8), so a kernel can give each XCD a
// fixed eighth of the weights, which then stays in that XCD's L2 while every
// token streams past it:
//
//   k_xcd_up    XCD r takes the TwELL tiles j = r, r + 8, ... of every token:
//               for each packed neuron n of tile j, h = a * <W_up[n, :], x_t>
//               (a from the pack), written to an h array shaped like the pack.
//               [Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷": only the
//               packed neurons' up rows are read.]
//   k_xcd_down  XCD r takes columns [r d / 8, (r + 1) d / 8) of y: for each
//               token, y[t, cols] = sum over its packed neurons of
//               h * W_down[cols, n] (W_down neuron-major), written once, in a
//               fixed order; no partial rows.
//
// Tokens whose pack overflows (a tile with more than E active neurons) are
// skipped; the dense backup computes their rows [same page, "Hybrid 應對非均勻
// 稀疏"]. The extra last workgroup of k_xcd_up routes the pack.
#include "common.cuh"
#include "kernels.cuh"
#include "route.cuh"
#include "wave.cuh"

namespace ffn {

constexpr int kXWaves = 4;
constexpr int kXTok = kXWaves;                         // tokens per workgroup, one per wave
constexpr int kXList = 1024;                           // list entries a wave holds in LDS

// ------------------------------------------------------------------ k_xcd_up
// A wave takes one token. One round of loads brings the token's tile counts,
// x_t (registers) and the indices and activations of its tile's E slots (lane
// s: slots s, s + 64); the entries are then processed in groups of RPG rows: the RPG rows' loads (CPL 16-byte chunks per lane each,
// a whole 1 KB contiguous per instruction) are issued together, the dot
// products with x_t (in registers, bf16 pairs through v_dot2c_f32_bf16) are
// reduced across the wave with the
// transpose reduction, and lane group r writes h of row r.
template <int CPL>
__global__ __launch_bounds__(64 * kXWaves) void k_xcd_up(const XcdDesc u) {
  constexpr int RPG = 16 / CPL > 0 ? 16 / CPL : 1;      // rows per group
  const int nchunks = (u.M + kXTok - 1) / kXTok;
  if ((int)blockIdx.x == 8 * nchunks) {
    if (u.route_pass) route_pass(u.route);
    return;
  }
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int xr = blockIdx.x & 7, chunk = blockIdx.x >> 3;
  const int d = u.d, T = u.T, E = u.E, ntiles = u.ntiles;
  const uint16_t* wup = reinterpret_cast<const uint16_t*>(u.w_up);
  const int t = chunk * kXTok + wave;
  if (t >= u.M) return;
  // one round of loads: the token's tile counts, x_t, and the slots of its
  // first tile in this XCD's class (all E slots, masked by the count after)
  const int cl = lane < ntiles ? u.cnt[(size_t)t * ntiles + lane] : 0;
  uint4 xv[CPL];
  const uint16_t* xrow = reinterpret_cast<const uint16_t*>(u.x) + (size_t)t * d + lane * 8;
#pragma unroll
  for (int k = 0; k < CPL; ++k) xv[k] = ldg16(xrow + k * 512);
  int nrn[2];
  float av[2];
  auto load_slots = [&](int j) {
    const size_t slot0 = ((size_t)t * ntiles + j) * E;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = lane + 64 * h;
      nrn[h] = s < E ? j * T + u.idx[slot0 + s] : 0;
      av[h] = s < E ? bf2f(reinterpret_cast<const uint16_t*>(u.val)[slot0 + s]) : 0.f;
    }
  };
  if (xr < ntiles) load_slots(xr);
  if (ballot64(lane < ntiles && cl > E) != 0ull) return;      // overflowing pack: dense backup
  for (int j = xr; j < ntiles; j += 8) {
    if (j != xr) load_slots(j);
    const size_t slot0 = ((size_t)t * ntiles + j) * E;
    const int c = wave_read(cl, j & 63);                       // j is wave-uniform
    for (int g0 = 0; g0 < c; g0 += RPG) {
      uint4 w[RPG][CPL];
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        const int s = g0 + r;
        const int n = wave_read((s >> 6) & 1 ? nrn[1] : nrn[0], s & 63);   // s is wave-uniform
        const uint16_t* row = wup + (size_t)n * d + lane * 8;
#pragma unroll
        for (int k = 0; k < CPL; ++k) w[r][k] = s < c ? ldg16(row + k * 512) : uint4{0, 0, 0, 0};
      }
      float v[RPG];
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) acc = dot8_bf_d2(w[r][k], xv[k], acc);
        v[r] = acc;
      }
      WaveTRed<RPG, 32>::run(v, lane);
      constexpr int SH = 6 - Log2<RPG>::value;
      const int r = lane >> SH, s = g0 + r;
      const float a = __shfl(av[(s >> 6) & 1], s & 63, FFN_WAVE);
      if ((lane & ((1 << SH) - 1)) == 0 && s < c) u.hp[slot0 + s] = a * v[0];
    }
  }
}

// ------------------------------------------------------------------ k_xcd_down
// A wave takes one token: it gathers the token's (neuron, h) list into its
// LDS (one round of loads over the pack's slots), then streams the
// neurons' W_down row slices: LPE lanes cover one row's d / 8 columns (16
// bytes each), so a load instruction covers 64 / LPE rows, and U instructions
// are in flight. The 64 / LPE row lanes are summed across the wave at the end.
// acc[k] summed over the lane bits from log2 O up (exact xor butterfly, in
// level order O, 2 O, .., 32).
template <int O>
__device__ __forceinline__ void xor_sum8(float (&acc)[8]) {
  if constexpr (O < 64) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += wave_xor<O>(acc[k]);
    xor_sum8<O * 2>(acc);
  }
}

template <int LPE>
__global__ __launch_bounds__(64 * kXWaves) void k_xcd_down(const XcdDesc u) {
  constexpr int EPI = 64 / LPE;                        // rows per load instruction
  constexpr int U = 16;                                // load instructions in flight
  __shared__ int s_n[kXWaves][kXList];
  __shared__ float s_h[kXWaves][kXList];
  __shared__ int s_ne[kXWaves];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int xr = blockIdx.x & 7, chunk = blockIdx.x >> 3;
  const int d = u.d, T = u.T, E = u.E, ntiles = u.ntiles, lgE = u.lg_e;
  const int sub = lane / LPE, q = lane % LPE;
  const int col = xr * (d / 8) + q * 8;
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(u.w_down_nm) + col;
  const int t = chunk * kXTok + wave;
  if (t >= u.M) return;
  {
    // one round of loads: tile counts (ntiles <= 64) and every slot of the
    // token's pack, kept when its position in the tile is below the count
    const int craw = lane < ntiles ? u.cnt[(size_t)t * ntiles + lane] : 0;
    const size_t tok0 = (size_t)t * ntiles * E;
    const int nz = ntiles << lgE;
    int nn[16];
    float hh[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int z = lane + 64 * i;
      nn[i] = z < nz ? (int)u.idx[tok0 + z] : 0;
      hh[i] = z < nz ? u.hp[tok0 + z] : 0.f;
    }
    if (ballot64(lane < ntiles && craw > E) != 0ull) return;  // overflowing pack: dense backup
    const int cl = min(craw, E);
    const int incl = wave_incl_scan(cl);
    const int pre = incl - cl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int z = lane + 64 * i;
      const int j = z >> lgE, s = z & (E - 1);
      const int cj = __shfl(cl, j & 63, FFN_WAVE), p = __shfl(pre, j & 63, FFN_WAVE) + s;
      if (z < nz && s < cj) {
        s_n[wave][p] = j * T + nn[i];
        s_h[wave][p] = hh[i];
      }
    }
    s_ne[wave] = wave_read(incl, 63);
  }
  __builtin_amdgcn_wave_barrier();
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  const int nl = s_ne[wave];
  for (int e0 = 0; e0 < nl; e0 += EPI * U) {
    uint4 w[U];
    float hv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int e = e0 + i * EPI + sub;
      const bool ok = e < nl;
      const int n = ok ? s_n[wave][e] : 0;
      hv[i] = ok ? s_h[wave][e] : 0.f;
      w[i] = ok ? ldg16(wd + (size_t)n * d) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float f[8];
      unpack8(w[i], f);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(hv[i], f[k], acc[k]);
    }
  }
  // sum the EPI row lanes (lane bits >= log2 LPE), in a fixed order
  xor_sum8<LPE>(acc);
  if (sub == 0) {
    uint4 out;
    out.x = f2bf(acc[0]) | (f2bf(acc[1]) << 16);
    out.y = f2bf(acc[2]) | (f2bf(acc[3]) << 16);
    out.z = f2bf(acc[4]) | (f2bf(acc[5]) << 16);
    out.w = f2bf(acc[6]) | (f2bf(acc[7]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(u.y) + (size_t)t * d + col) = out;
  }
}

// Shapes the XCD pair handles: bf16 ReLU packs (a in the pack), d a multiple of
// 512 up to 4096, at most 64 tiles, E a power of two up to 128, and every
// non-overflowing token's list within a wave's LDS.
bool xcd_ok(const XcdDesc& u) {
  // d / 512 must be 1, 2, 4 or 8: the widths the kernels are instantiated for
  const int dq = u.d / 512;
  if (u.M < 1 || u.d % 512 != 0 || u.d > 4096 || (dq & (dq - 1)) != 0 || u.ntiles < 1 || u.ntiles > 64 || u.E < 1 || u.E > 128 ||
      (u.E & (u.E - 1)) != 0 || (1 << u.lg_e) != u.E || u.ntiles * u.E > kXList)
    return false;
  return u.x && u.w_up && u.w_down_nm && u.cnt && u.idx && u.val && u.hp && u.y;
}

hipError_t launch_xcd_up(const XcdDesc& u, hipStream_t s) {
  if (!xcd_ok(u)) return hipErrorInvalidValue;
  const int nchunks = (u.M + kXTok - 1) / kXTok;
  const dim3 grid(8 * nchunks + 1), blk(64 * kXWaves);
  switch (u.d / 512) {
    case 1: ffn_launch(k_xcd_up<1>, grid, blk, 0, s, u); break;
    case 2: ffn_launch(k_xcd_up<2>, grid, blk, 0, s, u); break;
    case 4: ffn_launch(k_xcd_up<4>, grid, blk, 0, s, u); break;
    case 8: ffn_launch(k_xcd_up<8>, grid, blk, 0, s, u); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_xcd_down(const XcdDesc& u, hipStream_t s) {
  if (!xcd_ok(u)) return hipErrorInvalidValue;
  const int nchunks = (u.M + kXTok - 1) / kXTok;
  const dim3 grid(8 * nchunks), blk(64 * kXWaves);
  switch (u.d / 512) {
    case 1: ffn_launch(k_xcd_down<8>, grid, blk, 0, s, u); break;
    case 2: ffn_launch(k_xcd_down<16>, grid, blk, 0, s, u); break;
    case 4: ffn_launch(k_xcd_down<32>, grid, blk, 0, s, u); break;
    case 8: ffn_launch(k_xcd_down<64>, grid, blk, 0, s, u); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ffn
