// Decode path of the sparse gated FFN on gfx950: bf16 weights, at most 8
// tokens, ReLU gate with a bias or threshold selection.
//
// At a handful of tokens every product is a memory-bound weight stream
// (about one FLOP per byte), so the path is organised around reading each
// touched weight byte once, with all 256 CUs busy and every load of a wave
// issued before the first is used:
//
//   k_dec_lowrank  t = V x (low-rank gate only; LoPA page, "How LoPA Gating
//                  Restructures FFN Computation"): 1 KB pieces of V's rows,
//                  several per wave, reduced in LDS.
//   k_dec_gate     one workgroup per sub-tile of R gate rows (R divides the
//                  TwELL tile width T). The gate rows are streamed and dotted
//                  with every token; the epilogue applies the selection and
//                  writes the TwELL pack straight from LDS (Sparser/Faster/
//                  Lighter page, "TwELL 減掉轉換開銷"): a sub-tile learns its
//                  slot offset inside the TwELL tile from the counts the
//                  earlier sub-tiles publish (epoch-tagged words). Before it
//                  waits for those, the workgroup computes the up products of
//                  its neurons that are active for any token, u = <W_up[i,:], x>
//                  (each W_up row read once for all tokens), stores h = a * u
//                  in the dense hidden array h[token, neuron] and the
//                  sub-tile's union mask (one 64-bit word). A token
//                  whose tile overflows the ELL width still has every active
//                  neuron in the list, so no dense backup is needed at these
//                  token counts (Sparser/Faster/Lighter page, "Hybrid
//                  應對非均勻稀疏", routes busy rows; here they cost one more
//                  list entry per neuron).
//   k_dec_down     one workgroup per 16-byte column chunk of y: it reads the
//                  union masks in one round, deals their set bits to its
//                  threads (prefix of popcounts in LDS), then reads h and the
//                  rows in a second round and accumulates h * W_down^T[i, chunk]
//                  for every token, reduces across its lanes in a fixed
//                  order and writes y once. No partial rows, no atomics, and
//                  the result is bitwise reproducible. The eight chunks of a
//                  128-byte line go to the same XCD (workgroups are dealt to
//                  the eight XCDs round-robin), so its L2 serves the line to
//                  all of them. An extra workgroup routes the pack.
#include <algorithm>
#include <type_traits>

#include "common.cuh"
#include "kernels.cuh"
#include "route.cuh"

namespace ffn {

// ------------------------------------------------------------------ wave transpose reduction
// Reduces N values per lane across the 64 lanes of a wave. Each halving step
// keeps one half of the values and swaps the other half with the partner lane,
// so N - 1 + (6 - log2 N) shuffles replace N full butterflies. Afterwards
// v[0] of lane L holds the wave total of value index L >> (6 - log2 N).
template <int N, int O>
struct WaveTRed {
  template <int V>
  __device__ __forceinline__ static void run(float (&v)[V], int lane) {
    const bool upper = (lane & O) != 0;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      const float lo = v[j], hi = v[j + N / 2];
      const float keep = upper ? hi : lo;
      const float send = upper ? lo : hi;
      v[j] = keep + __shfl_xor(send, O, FFN_WAVE);
    }
    WaveTRed<N / 2, O / 2>::run(v, lane);
  }
};
template <int O>
struct WaveTRed<1, O> {
  template <int V>
  __device__ __forceinline__ static void run(float (&v)[V], int lane) {
    v[0] += __shfl_xor(v[0], O, FFN_WAVE);
    WaveTRed<1, O / 2>::run(v, lane);
  }
};
template <>
struct WaveTRed<1, 0> {
  template <int V>
  __device__ __forceinline__ static void run(float (&)[V], int) {}
};
template <int N>
struct Log2 {
  static constexpr int value = N <= 1 ? 0 : 1 + Log2<N / 2>::value;
};
template <>
struct Log2<1> {
  static constexpr int value = 0;
};

// dot of 8 bf16 weights with 8 bf16 inputs (fp32 products, fixed order)
__device__ __forceinline__ float dot8_bf(const uint4 a, const uint4 b, float acc) {
  float fa[8], fb[8];
  unpack8(a, fa);
  unpack8(b, fb);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc = fmaf(fa[k], fb[k], acc);
  return acc;
}
__device__ __forceinline__ float dot8_f32(const uint4 a, const float4 b0, const float4 b1, float acc) {
  float fa[8];
  unpack8(a, fa);
  acc = fmaf(fa[0], b0.x, acc); acc = fmaf(fa[1], b0.y, acc);
  acc = fmaf(fa[2], b0.z, acc); acc = fmaf(fa[3], b0.w, acc);
  acc = fmaf(fa[4], b1.x, acc); acc = fmaf(fa[5], b1.y, acc);
  acc = fmaf(fa[6], b1.z, acc); acc = fmaf(fa[7], b1.w, acc);
  return acc;
}

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

// Stages `rows` rows of `cols16` 16-byte chunks (row stride ld16 chunks in
// global memory) into LDS, zero-filling rows [rows, MAXM).
template <int MAXM>
__device__ __forceinline__ void stage_rows(uint4* dst, const uint4* src, int rows, int cols16, size_t ld16) {
  for (int p = threadIdx.x; p < MAXM * cols16; p += blockDim.x) {
    const int m = p / cols16, c = p - m * cols16;
    dst[p] = m < rows ? src[(size_t)m * ld16 + c] : uint4{0, 0, 0, 0};
  }
}

// ------------------------------------------------------------------ k_dec_lowrank
template <int IPW, int MAXM>
__global__ __launch_bounds__(64 * kDecVWaves) void k_dec_lowrank(const DecodeDesc d) {
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

// ------------------------------------------------------------------ k_dec_gate
__device__ __forceinline__ float dec_bias(const DecodeDesc& d, int t) { return d.bias ? d.bias[t] : d.bias_scalar; }
__device__ __forceinline__ float dec_cut(const DecodeDesc& d, int t) {
  return d.sel == SEL_THRESH ? fmaxf(d.tau[t], 0.f) : 0.f;
}

// Waits until an epoch-tagged look-back word carries this pass's epoch and
// returns its count.
__device__ __forceinline__ int lb_count(const uint64_t* p, uint32_t epoch, uint64_t first) {
  uint64_t w = first;
  while ((uint32_t)(w >> 32) != epoch) {
    __builtin_amdgcn_s_sleep(1);
    w = load64_relaxed(p);
  }
  return (int)(uint32_t)w;
}

template <int NW, int IPW, int MAXM, bool LOWRANK, int MODE>
__global__ __launch_bounds__(64 * NW) void k_dec_gate(const DecodeDesc d) {
  constexpr bool PART = MODE == DEC_PART;
  extern __shared__ uint4 s_dyn[];
  __shared__ float s_part[NW * IPW * MAXM];
  __shared__ float s_g[64 * MAXM];
  __shared__ uint64_t s_bal[MAXM];
  __shared__ int s_urow[64];
  __shared__ float s_h[PART ? 64 * MAXM : 1];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int M = d.M, dm = d.d, F = d.F;
  const int K = d.K;
  int P = 1;
  while (P * 512 < K) P <<= 1;
  const int R = NW * IPW / P;
  const int sub = blockIdx.x, n0 = sub * R;
  uint16_t* s_x = reinterpret_cast<uint16_t*>(s_dyn);                               // [MAXM x d] bf16
  float* s_t = reinterpret_cast<float*>(reinterpret_cast<char*>(s_dyn) + (size_t)MAXM * dm * 2);  // [MAXM x rank]

  // ---- gate row loads first; the token inputs are staged while they fly
  uint4 a[IPW];
  dec_gemv_issue<NW, IPW>(reinterpret_cast<const uint16_t*>(d.a_gate), F, K, P, n0, a);
  stage_rows<MAXM>(s_dyn, reinterpret_cast<const uint4*>(d.x), M, dm / 8, dm / 8);
  if (LOWRANK)
    stage_rows<MAXM>(reinterpret_cast<uint4*>(s_t), reinterpret_cast<const uint4*>(d.t), M, d.rank / 4, d.rank / 4);
  const uint32_t epoch = __hip_atomic_load(&d.ctrl[CTRL_EPOCH], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  __syncthreads();
  dec_gemv_finish<NW, IPW, MAXM, LOWRANK>(a, K, P, s_x, s_t, s_part, s_g);

  // ---- selection: one wave per token; the sub-tile's mask is one ballot (R <= 64)
  const int T = d.T, Q = T / R, q = (n0 % T) / R, j = n0 / T;
  const int ntiles = F / T, nsub = F / R;
  if (wave < M) {
    const int m = wave;
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
  }
  if (threadIdx.x < MAXM && threadIdx.x >= M) s_bal[threadIdx.x] = 0ull;
  __syncthreads();

  // first read of the earlier sub-tiles' counts of tile j (per token), while
  // this workgroup's up products run
  const bool tok_wave = wave < M && Q > 1;
  const uint64_t* twp = d.lb + (size_t)(tok_wave ? wave : 0) * nsub + (size_t)j * Q + lane;
  uint64_t tw = 0;
  if (tok_wave && lane < q) tw = load64_relaxed(twp);

  // ---- up products of the neurons active for any token: h = a * <W_up[i,:], x>
  if (d.up) {
    uint64_t uni = 0ull;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) uni |= s_bal[m];
    const int nu = __popcll(uni);
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
        for (int k = k0 + wave; k < min(nu, k0 + DB); k += NW) up_row(k, true);
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

  // ---- TwELL pack: this sub-tile's entries at their offset inside tile j
  if (wave < M) {
    const int m = wave;
    const uint64_t bal = s_bal[m];
    int pre = 0;
    if (Q > 1) pre = wave_sum_i(lane < q ? lb_count(twp, epoch, tw) : 0);
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
  }
}

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
// row: 8 threads read one partial row's slice (16 bytes each), 32 rows in
// flight per pass; the 32 row sums per column are then added in row order.
constexpr int kRedThreads = 256;

template <int MAXM>
__global__ __launch_bounds__(kRedThreads) void k_dec_reduce(const DecodeDesc d) {
  constexpr int B = 16 / MAXM;                          // partial rows in flight per thread and token
  __shared__ int s_list[kDecMaxSub];
  __shared__ int s_scan[kRedThreads / 64];
  __shared__ float s_red[MAXM][32][33];
  const int nsl = d.d / 32;
  if (d.route_pass && (int)blockIdx.x == nsl) {
    route_pass(d.route);
    return;
  }
  const int tid = threadIdx.x, q = tid & 7, r = tid >> 3;
  const int sl = blockIdx.x, M = d.M, dm = d.d, nsub = d.F / d.R;
  // ascending list of the sub-tiles that wrote a partial row
  const int per = (nsub + kRedThreads - 1) / kRedThreads;
  const int s0 = min(nsub, tid * per), s1 = min(nsub, s0 + per);
  int loc = 0;
  for (int s = s0; s < s1; ++s) loc += d.umask[s] != 0ull;
  int ne;
  int pos = block_excl_scan<kRedThreads>(loc, s_scan, &ne);
  for (int s = s0; s < s1; ++s)
    if (d.umask[s] != 0ull) s_list[pos++] = s;
  __syncthreads();

  float acc[MAXM][4];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[m][k] = 0.f;
  const size_t col = (size_t)sl * 32 + q * 4;
  for (int p0 = r; p0 < ne; p0 += 32 * B) {
    float4 v[B][MAXM];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int p = p0 + 32 * i;
      const int s = p < ne ? s_list[p] : 0;
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        v[i][m] = (p < ne && m < M) ? *reinterpret_cast<const float4*>(d.part + ((size_t)s * M + m) * dm + col)
                                    : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < B; ++i)
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        acc[m][0] += v[i][m].x;
        acc[m][1] += v[i][m].y;
        acc[m][2] += v[i][m].z;
        acc[m][3] += v[i][m].w;
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

// ------------------------------------------------------------------ k_dec_up (split mode)
// The union neurons (set bits of the sub-tile masks, ascending) are dealt to a
// fixed grid in equal contiguous ranges; a wave takes two neurons at a time
// (16 row loads per lane in flight): u = <W_up[n,:], x_t> for every token,
// h = a * u (a from the gate kernel). Writes the compact list (neuron, h per
// token) in union order and its length.
constexpr int kUpWaves = 8;
constexpr int kUpGrid = 512;

template <int MAXM>
__device__ __forceinline__ void up_dot_store(const DecodeDesc& d, const uint4 (&w)[8], int pd, const uint16_t* s_x,
                                             int n, int e, int lane) {
  const int M = d.M, dm = d.d;
  float a[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) a[m] = m < M ? d.ad[(size_t)m * d.F + n] : 0.f;
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
    float am = a[0];
#pragma unroll
    for (int q = 1; q < MAXM; ++q)
      if (q == m) am = a[q];
    d.ul_h[(size_t)e * kDecMaxM + m] = m < M ? am * v[0] : 0.f;
  }
  if (lane == 0) d.ul_nrn[e] = n;
}

template <int MAXM>
__global__ __launch_bounds__(64 * kUpWaves) void k_dec_up(const DecodeDesc d) {
  extern __shared__ uint4 s_dyn[];
  __shared__ uint64_t s_mask[kDecMaxSub];
  __shared__ int s_pre[kDecMaxSub + 1];
  __shared__ int s_scan[kUpWaves];
  uint16_t* s_x = reinterpret_cast<uint16_t*>(s_dyn);       // [MAXM x d]
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int M = d.M, dm = d.d, F = d.F, R = d.R, nsub = F / R;
  constexpr int NT = 64 * kUpWaves;
  const int per = (nsub + NT - 1) / NT;
  const int s0 = min(nsub, tid * per), s1 = min(nsub, s0 + per);
  int loc = 0;
  for (int s = s0; s < s1; ++s) {
    const uint64_t w = d.umask[s];
    s_mask[s] = w;
    loc += __popcll(w);
  }
  stage_rows<MAXM>(s_dyn, reinterpret_cast<const uint4*>(d.x), M, dm / 8, dm / 8);
  int total;
  int run = block_excl_scan<NT>(loc, s_scan, &total);
  for (int s = s0; s < s1; ++s) {
    s_pre[s] = run;
    run += __popcll(s_mask[s]);
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) *d.ul_total = total;
  const int e0 = (int)((long long)total * blockIdx.x / gridDim.x);
  const int e1 = (int)((long long)total * (blockIdx.x + 1) / gridDim.x);
  const int pd = (dm + 511) / 512;
  auto neuron_of = [&](int e) {
    int lo = 0, hi = nsub - 1;                     // last sub-tile with s_pre <= e
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= e) lo = mid;
      else hi = mid - 1;
    }
    return lo * R + nth_set_bit(s_mask[lo], e - s_pre[lo]);
  };
  for (int ea = e0 + wave; ea < e1; ea += 2 * kUpWaves) {
    const int eb = ea + kUpWaves;
    const bool hb = eb < e1;
    const int na = neuron_of(ea), nb = hb ? neuron_of(eb) : 0;
    const uint16_t* ra = reinterpret_cast<const uint16_t*>(d.w_up) + (size_t)na * dm;
    const uint16_t* rb = reinterpret_cast<const uint16_t*>(d.w_up) + (size_t)nb * dm;
    uint4 wa[8], wb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = c * 512 + lane * 8;
      const bool ok = c < pd && col < dm;
      wa[c] = ok ? ldg16(ra + col) : uint4{0, 0, 0, 0};
      wb[c] = (ok && hb) ? ldg16(rb + col) : uint4{0, 0, 0, 0};
    }
    up_dot_store<MAXM>(d, wa, pd, s_x, na, ea, lane);
    if (hb) up_dot_store<MAXM>(d, wb, pd, s_x, nb, eb, lane);
  }
}

// ------------------------------------------------------------------ k_dec_down2 (split mode)
// One workgroup per slice of LW 16-byte chunks of y's columns (LW = 4 or 8:
// 64 or 128 bytes of every row). Its 1024 threads form 1024 / LW row lanes:
// lane q of a row lane reads chunk q of the slice, so a wave reads 64 / LW
// whole row slices per instruction. Row lane r takes list entries r, r + RL,
// ...; the list length is read in the same round as the first entries (slots
// past it hold stale but valid neuron ids and are masked). Sums over the row
// lanes are reduced across the wave (WaveTRed over the row-lane bits) and then
// across the waves in order; the extra last workgroup routes the pack.
constexpr int kDown2Threads = 256;

// Halving steps of WaveTRed restricted to the lane bits >= OMIN. With H the
// number of halving steps (log2 V, at most 6 - log2 OMIN), each lane keeps
// V >> H values with index base (lane >> (6 - H)) * (V >> H), summed over the
// lanes that share lane % OMIN.
template <int N, int O, int OMIN>
struct WaveTRedHi {
  template <int V>
  __device__ __forceinline__ static void run(float (&v)[V], int lane) {
    if constexpr (O >= OMIN) {
      if constexpr (N > 1) {
        const bool upper = (lane & O) != 0;
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
          const float lo = v[j], hi = v[j + N / 2];
          const float keep = upper ? hi : lo;
          const float send = upper ? lo : hi;
          v[j] = keep + __shfl_xor(send, O, FFN_WAVE);
        }
        WaveTRedHi<N / 2, O / 2, OMIN>::run(v, lane);
      } else {
        v[0] += __shfl_xor(v[0], O, FFN_WAVE);
        WaveTRedHi<1, O / 2, OMIN>::run(v, lane);
      }
    }
  }
};

template <int MAXM>
__global__ __launch_bounds__(kDown2Threads) void k_dec_down2(const DecodeDesc d) {
  constexpr int LW = 8;                                 // 16-byte chunks per slice (128 bytes)
  constexpr int NW = kDown2Threads / 64, RL = kDown2Threads / LW;
  constexpr int B = MAXM <= 2 ? 8 : 4;                  // entries in flight per thread
  constexpr int V = 8 * MAXM;                           // sums per thread
  constexpr int STEPS = 6 - Log2<LW>::value;            // row-lane bits of a wave
  constexpr int H = Log2<V>::value < STEPS ? Log2<V>::value : STEPS;   // halving steps
  constexpr int KEEP = V >> H;                          // sums each lane keeps
  __shared__ float s_red[NW][LW][V];
  const int nsl = d.d / (8 * LW), S = d.ngroups;
  const int lane = lane_id(), wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int q = tid % LW, rl = tid / LW;
  const int b = blockIdx.x, g = b % S, sl = b / S;     // the S groups of a slice are neighbours
  const int M = d.M, F = d.F;
  const uint16_t* wd = reinterpret_cast<const uint16_t*>(d.w_down_nm) + (size_t)sl * 8 * LW + q * 8;
  float acc[MAXM][8];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[m][k] = 0.f;
  // entries g + S * (rl + RL * i): the list length is read in the same round
  // as the first entries (slots past it hold stale but valid ids, masked)
  int total = F;
  for (int j0 = rl; g + S * j0 < total; j0 += RL * B) {
    int nrn[B];
    float h[B][MAXM];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int e = g + S * (j0 + RL * i);
      nrn[i] = e < F ? d.ul_nrn[e] : 0;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) h[i][m] = (e < F && m < M) ? d.ul_h[(size_t)e * kDecMaxM + m] : 0.f;
    }
    if (j0 == rl) total = *d.ul_total;
    uint4 w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int e = g + S * (j0 + RL * i);
      w[i] = e < total ? ldg16(wd + (size_t)nrn[i] * d.d) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int e = g + S * (j0 + RL * i);
      if (e < total) {
        float f[8];
        unpack8(w[i], f);
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[m][k] = fmaf(h[i][m], f[k], acc[m][k]);
      }
    }
  }
  float v[V];
#pragma unroll
  for (int m = 0; m < MAXM; ++m)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[m * 8 + k] = acc[m][k];
  WaveTRedHi<V, 32, LW>::run(v, lane);
  {
    const int base = (lane >> (6 - H)) * KEEP;         // value indices this lane holds
    if (base < V) {
#pragma unroll
      for (int j = 0; j < KEEP; ++j) s_red[wave][q][base + j] = v[j];
    }
  }
  __syncthreads();
  for (int o = tid; o < LW * V; o += kDown2Threads) {
    const int qq = o / V, j = o % V, m = j / 8, k = j % 8;
    float s = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) s += s_red[w2][qq][j];
    if (m < M) d.part[((size_t)g * M + m) * d.d + (size_t)sl * 8 * LW + qq * 8 + k] = s;
  }
}

// y = sum of the S group partials in group order; the extra last workgroup
// routes the pack.
__global__ __launch_bounds__(256) void k_dec_reduce2(const DecodeDesc d) {
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

// ------------------------------------------------------------------ launches
static int pow2_pieces(int K) {
  int P = 1;
  while (P * 512 < K) P <<= 1;
  return P;
}

static int dec_maxm(int M) { return M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8)); }

size_t dec_lowrank_lds(const DecodeDesc& d) { return (size_t)dec_maxm(d.M) * d.d * 2; }
size_t dec_gate_lds(const DecodeDesc& d) {
  return (size_t)dec_maxm(d.M) * d.d * 2 + (d.rank ? (size_t)dec_maxm(d.M) * d.rank * 4 : 0);
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
  DecodeDesc e = d;
  e.ipw = pow2_pieces(d.d);
  if (e.ipw > 8) return hipErrorInvalidValue;
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
  // a pack-only pass (no hidden values) uses the chunk-mode kernel with up = 0
  const int mode = d.up ? d.mode : DEC_CHUNK;
  if (mode == DEC_PART) return go_gate_k<IPW, MAXM, LOWRANK, DEC_PART>(d, s);
  if (mode == DEC_SPLIT) return go_gate_k<IPW, MAXM, LOWRANK, DEC_SPLIT>(d, s);
  return go_gate_k<IPW, MAXM, LOWRANK, DEC_CHUNK>(d, s);
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
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dec_gate(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM) return hipErrorInvalidValue;
  const int P = pow2_pieces(d.K);
  if (dec_gate_waves(dec_maxm(d.M)) * d.ipw != d.R * P || d.R > 64 || d.R < 2 || d.T % d.R != 0 || d.F % d.R != 0 || d.T / d.R > 64)
    return hipErrorInvalidValue;
  switch (dec_maxm(d.M)) {
    case 1: return go_gate_m<1>(d, s);
    case 2: return go_gate_m<2>(d, s);
    case 4: return go_gate_m<4>(d, s);
    default: return go_gate_m<8>(d, s);
  }
}

hipError_t launch_dec_reduce(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || d.d % 32 != 0 || d.F / d.R > kDecMaxSub || !d.part) return hipErrorInvalidValue;
  const dim3 grid(d.d / 32 + (d.route_pass ? 1 : 0)), blk(kRedThreads);
  switch (dec_maxm(d.M)) {
    case 1: ffn_launch((k_dec_reduce<1>), grid, blk, 0, s, d); break;
    case 2: ffn_launch((k_dec_reduce<2>), grid, blk, 0, s, d); break;
    case 4: ffn_launch((k_dec_reduce<4>), grid, blk, 0, s, d); break;
    default: ffn_launch((k_dec_reduce<8>), grid, blk, 0, s, d); break;
  }
  return hipGetLastError();
}

size_t dec_up_lds(const DecodeDesc& d) { return (size_t)dec_maxm(d.M) * d.d * 2; }

template <int MAXM>
static hipError_t go_up(const DecodeDesc& d, hipStream_t s) {
  const size_t lds = dec_up_lds(d);
  hipError_t e = lds_attr(k_dec_up<MAXM>, lds);
  if (e != hipSuccess) return e;
  ffn_launch((k_dec_up<MAXM>), dim3(kUpGrid), dim3(64 * kUpWaves), lds, s, d);
  return hipGetLastError();
}

hipError_t launch_dec_up(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || d.F / d.R > kDecMaxSub || !d.ad || !d.ul_nrn || !d.ul_h || !d.ul_total)
    return hipErrorInvalidValue;
  switch (dec_maxm(d.M)) {
    case 1: return go_up<1>(d, s);
    case 2: return go_up<2>(d, s);
    case 4: return go_up<4>(d, s);
    default: return go_up<8>(d, s);
  }
}

int dec_down2_groups(int d_model) { return std::max(1, std::min(32, 1024 / (d_model / 64))); }

hipError_t launch_dec_down2(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || d.d % 64 != 0 || !d.ul_nrn || !d.ul_h || !d.ul_total || !d.part ||
      d.ngroups != dec_down2_groups(d.d))
    return hipErrorInvalidValue;
  const dim3 grid(d.d / 64 * d.ngroups), blk(kDown2Threads);
  switch (dec_maxm(d.M)) {
    case 1: ffn_launch((k_dec_down2<1>), grid, blk, 0, s, d); break;
    case 2: ffn_launch((k_dec_down2<2>), grid, blk, 0, s, d); break;
    case 4: ffn_launch((k_dec_down2<4>), grid, blk, 0, s, d); break;
    default: ffn_launch((k_dec_down2<8>), grid, blk, 0, s, d); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = d.M * d.d;
  ffn_launch(k_dec_reduce2, dim3((n + 1023) / 1024 + (d.route_pass ? 1 : 0)), dim3(256), 0, s, d);
  return hipGetLastError();
}

int dec_rows_per_wg(int K, int T, int m, int* ipw_out) {
  const int P = pow2_pieces(K);
  if (P > 8 || m < 1 || m > kDecMaxM) return 0;
  const int nw = dec_gate_waves(dec_maxm(m));
  for (int ipw = 4; ipw >= 1; ipw >>= 1) {
    const int R = nw * ipw / P;
    if (R >= 2 && R <= 64 && T % R == 0 && T / R <= 64) {
      if (ipw_out) *ipw_out = ipw;
      return R;
    }
  }
  return 0;
}

hipError_t launch_dec_down(const DecodeDesc& d, hipStream_t s) {
  if (d.M < 1 || d.M > kDecMaxM || d.d % 64 != 0 || d.F / d.R > kDecMaxSub) return hipErrorInvalidValue;
  const dim3 grid(d.d / 8 + (d.route_pass ? 1 : 0)), blk(kDownThreads);
  switch (dec_maxm(d.M)) {
    case 1: ffn_launch((k_dec_down<1>), grid, blk, 0, s, d); break;
    case 2: ffn_launch((k_dec_down<2>), grid, blk, 0, s, d); break;
    case 4: ffn_launch((k_dec_down<4>), grid, blk, 0, s, d); break;
    default: ffn_launch((k_dec_down<8>), grid, blk, 0, s, d); break;
  }
  return hipGetLastError();
}

}  // namespace ffn
