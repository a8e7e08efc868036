// Backward pass of the sparse gated FFN on gfx950 (full-rank ReLU gate, bias
// or threshold selection, the forward pass's selection held fixed).
// Source: Sparser/Faster/Lighter page, section "Hybrid 應對非均勻稀疏": in
// training, most tokens keep their activations in the compact format and the
// few busy ones go through a dense backup, which cuts dense work and stored
// activations. Here the forward pass's TwELL pack is the stored state of the
// compact tokens (activation a = z of each active neuron); a routed (busy)
// token's gate row is recomputed densely (a matrix-core GEMM over the dense
// list, before these kernels) and its active neurons are taken from it.
//
// With dh = W_down^T dy: du = dh a, dz = dh u (active entries), h = a u,
// dW_down[:, i] += sum_t h dy_t, dW_up[i, :] += sum_t du x_t,
// dW_gate[i, :] += sum_t dz x_t, dx_t = sum_i du W_up[i, :] + dz W_gate[i, :].
//
//   k_bw_slots   dense-list slot of every routed token (a block scan).
//   k_bw_count   per (TwELL tile, block of 64 tokens): pairs per neuron.
//   k_bw_offsets per neuron: offsets of its pairs per token block, and its total.
//   k_bw_colptr  exclusive scan of the neuron totals.
//   k_bw_fill    per (tile, token block): the neuron-major pair list, tokens in
//                order (deterministic sums below).
//   k_bw_neuron  one workgroup per active neuron: its W_up and W_down rows once
//                in registers, its tokens four at a time (u and dh by block
//                reduction, then du, dz, h), the three gradient rows summed in
//                token order and added to the fp32 accumulators.
//   k_bw_dx      one workgroup per token: dx from its active neurons' W_up and
//                W_gate rows and their du, dz.
//   k_bw_duz     training batch sizes: each token's du and dz as one dense bf16
//                row (du over the neurons, then dz), so that dx is a
//                matrix-core GEMM with [W_up; W_gate] transposed: at 10%
//                density the per-token row gathers cost more than the dense
//                product.
#include <algorithm>

#include "common.cuh"
#include "kernels.cuh"
#include "wave.cuh"

namespace ffn {

namespace {

constexpr int kBwThreads = 256;
constexpr int kBwChunks = 2;       // 8-element chunks of a d-row per thread at most (d <= 4096)
constexpr int kBwBatch = 4;        // pairs per batch in the neuron and dx kernels

__device__ __forceinline__ float bw_bias(const BwDesc& d, int t) { return d.bias ? d.bias[t] : d.bias_scalar; }
__device__ __forceinline__ float bw_cut(const BwDesc& d, int t) {
  return d.sel == SEL_THRESH ? fmaxf(d.tau[t], 0.f) : 0.f;
}

// 8 consecutive elements kept in their storage form (bf16: one 16-byte
// chunk, 4 registers; fp32: two float4) and unpacked where used, so that a
// batch of rows in flight costs half the registers.
template <bool BF>
struct Raw8;
template <>
struct Raw8<true> {
  uint4 v;
  __device__ __forceinline__ void load(const void* base, size_t off, bool ok) {
    v = ok ? ldg16(static_cast<const uint16_t*>(base) + off) : uint4{0, 0, 0, 0};
  }
  __device__ __forceinline__ void get(float (&f)[8]) const { unpack8(v, f); }
};
template <>
struct Raw8<false> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, size_t off, bool ok) {
    const float* p = static_cast<const float*>(base) + off;
    a = ok ? *reinterpret_cast<const float4*>(p) : float4{0.f, 0.f, 0.f, 0.f};
    b = ok ? *reinterpret_cast<const float4*>(p + 4) : float4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void get(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// activation value a of pair position p (token t)
__device__ __forceinline__ float bw_a(const BwDesc& d, long long p, int t) {
  if (p >= d.pbase) return d.zr[p - d.pbase] + bw_bias(d, t);
  if (d.dtype == DT_BF16) return bf2f(static_cast<const uint16_t*>(d.val)[p]);
  return static_cast<const float*>(d.val)[p];
}

}  // namespace

// ------------------------------------------------------------------ slots of routed tokens
__global__ __launch_bounds__(1024) void k_bw_slots(const BwDesc d) {
  __shared__ int s_scan[16];
  int carry = 0;
  for (int t0 = 0; t0 < d.m; t0 += 1024) {
    const int t = t0 + threadIdx.x;
    const int f = (t < d.m && d.route[t]) ? 1 : 0;
    int tot = 0;
    const int ex = block_excl_scan<1024>(f, s_scan, &tot);
    if (t < d.m) d.slot_of[t] = f ? carry + ex : -1;
    carry += tot;
  }
}

// ------------------------------------------------------------------ neuron-major pair index
__global__ __launch_bounds__(kBwThreads) void k_bw_count(const BwDesc d) {
  __shared__ int s_c[1024];
  const int j = blockIdx.x, nb = blockIdx.y;
  for (int i = threadIdx.x; i < d.T; i += kBwThreads) s_c[i] = 0;
  __syncthreads();
  const int t1 = min(d.m, (nb + 1) * kBwBlock);
  for (int t = nb * kBwBlock; t < t1; ++t) {
    const int r = d.slot_of[t];
    if (r < 0) {
      const size_t pk = (size_t)t * d.ntiles + j;
      const int n = min(d.cnt[pk], d.E);
      for (int s = threadIdx.x; s < n; s += kBwThreads) atomicAdd(&s_c[d.idx[pk * d.E + s]], 1);
    } else {
      const float b = bw_bias(d, t), cut = bw_cut(d, t);
      for (int i = threadIdx.x; i < d.T; i += kBwThreads)
        if (d.zr[(size_t)r * d.F + j * d.T + i] + b > cut) atomicAdd(&s_c[i], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d.T; i += kBwThreads) d.blk[(size_t)nb * d.F + j * d.T + i] = s_c[i];
}

// per neuron: counts per token block -> offsets within the neuron; total -> colptr[i]
__global__ __launch_bounds__(kBwThreads) void k_bw_offsets(const BwDesc d) {
  const int i = blockIdx.x * kBwThreads + threadIdx.x;
  if (i >= d.F) return;
  int run = 0;
  for (int nb = 0; nb < d.nblk; ++nb) {
    int* c = d.blk + (size_t)nb * d.F + i;
    const int v = *c;
    *c = run;
    run += v;
  }
  d.colptr[i] = run;
}

__global__ __launch_bounds__(1024) void k_bw_colptr(const BwDesc d) {
  __shared__ int s_scan[16];
  int carry = 0;
  for (int i0 = 0; i0 < d.F; i0 += 1024) {
    const int i = i0 + threadIdx.x;
    const int v = i < d.F ? d.colptr[i] : 0;
    int tot = 0;
    const int ex = block_excl_scan<1024>(v, s_scan, &tot);
    if (i < d.F) d.colptr[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) d.colptr[d.F] = carry;
}

__global__ __launch_bounds__(kBwThreads) void k_bw_fill(const BwDesc d) {
  __shared__ int s_pos[1024];
  const int j = blockIdx.x, nb = blockIdx.y;
  for (int i = threadIdx.x; i < d.T; i += kBwThreads)
    s_pos[i] = d.colptr[j * d.T + i] + d.blk[(size_t)nb * d.F + j * d.T + i];
  __syncthreads();
  const int t1 = min(d.m, (nb + 1) * kBwBlock);
  for (int t = nb * kBwBlock; t < t1; ++t) {
    const int r = d.slot_of[t];
    if (r < 0) {
      const size_t pk = (size_t)t * d.ntiles + j;
      const int n = min(d.cnt[pk], d.E);
      for (int s = threadIdx.x; s < n; s += kBwThreads) {
        const int q = s_pos[d.idx[pk * d.E + s]]++;
        d.ent_tok[q] = t;
        d.ent_pos[q] = (int32_t)(pk * d.E + s);
      }
    } else {
      const float b = bw_bias(d, t), cut = bw_cut(d, t);
      for (int i = threadIdx.x; i < d.T; i += kBwThreads) {
        const size_t zi = (size_t)r * d.F + j * d.T + i;
        if (d.zr[zi] + b > cut) {
          const int q = s_pos[i]++;
          d.ent_tok[q] = t;
          d.ent_pos[q] = (int32_t)(d.pbase + (long long)zi);
        }
      }
    }
    __syncthreads();                               // a neuron's counter may move to another thread next token
  }
}

// ------------------------------------------------------------------ per neuron: du, dz, weight gradients
// CH: 8-element chunks of a d-row per thread (d <= 2048 * CH).
template <bool BF, int CH>
__global__ __launch_bounds__(kBwThreads) void k_bw_neuron(const BwDesc d) {
  __shared__ float s_red[4][2 * kBwBatch];
  const int i = blockIdx.x;
  const int q0 = d.colptr[i], q1 = d.colptr[i + 1];
  if (q0 == q1) return;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  Raw8<BF> wu[CH], wd[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (threadIdx.x + c * kBwThreads) * 8;
    wu[c].load(d.w_up, (size_t)i * d.d + col, col < d.d);
    wd[c].load(d.w_down_nm, (size_t)i * d.d + col, col < d.d);
  }
  float gu[CH][8], gg[CH][8], gd[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) gu[c][e] = gg[c][e] = gd[c][e] = 0.f;

  for (int qb = q0; qb < q1; qb += kBwBatch) {
    Raw8<BF> xv[kBwBatch][CH], yv[kBwBatch][CH];
#pragma unroll
    for (int b = 0; b < kBwBatch; ++b) {
      const bool live = qb + b < q1;
      const int t = live ? d.ent_tok[qb + b] : 0;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int col = (threadIdx.x + c * kBwThreads) * 8;
        xv[b][c].load(d.x, (size_t)t * d.d + col, live && col < d.d);
        yv[b][c].load(d.dy, (size_t)t * d.d + col, live && col < d.d);
      }
    }
    float part[2 * kBwBatch];
#pragma unroll
    for (int b = 0; b < kBwBatch; ++b) {
      float su = 0.f, sh = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float w8[8], v8[8];
        wu[c].get(w8);
        xv[b][c].get(v8);
#pragma unroll
        for (int e = 0; e < 8; ++e) su = fmaf(w8[e], v8[e], su);
        wd[c].get(w8);
        yv[b][c].get(v8);
#pragma unroll
        for (int e = 0; e < 8; ++e) sh = fmaf(w8[e], v8[e], sh);
      }
      part[b] = su;
      part[kBwBatch + b] = sh;
    }
    WaveTRed<2 * kBwBatch, 32>::run(part, lane);
    constexpr int SH = 6 - Log2<2 * kBwBatch>::value;
    if ((lane & ((1 << SH) - 1)) == 0) s_red[wave][lane >> SH] = part[0];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kBwBatch; ++b) {
      if (qb + b >= q1) break;
      const float u = ((s_red[0][b] + s_red[1][b]) + s_red[2][b]) + s_red[3][b];
      const float dh = ((s_red[0][kBwBatch + b] + s_red[1][kBwBatch + b]) + s_red[2][kBwBatch + b]) +
                       s_red[3][kBwBatch + b];
      const int t = d.ent_tok[qb + b];
      const long long p = d.ent_pos[qb + b];
      const float a = bw_a(d, p, t);
      const float du = dh * a, dz = dh * u, h = a * u;
      if (threadIdx.x == 0) {
        d.du[p] = du;
        d.dz[p] = dz;
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float x8[8], y8[8];
        xv[b][c].get(x8);
        yv[b][c].get(y8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gu[c][e] = fmaf(du, x8[e], gu[c][e]);
          gg[c][e] = fmaf(dz, x8[e], gg[c][e]);
          gd[c][e] = fmaf(h, y8[e], gd[c][e]);
        }
      }
    }
    __syncthreads();                               // s_red is rewritten by the next batch
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (threadIdx.x + c * kBwThreads) * 8;
    if (col >= d.d) continue;
    const size_t o = (size_t)i * d.d + col;
    auto add8 = [&](float* dst, const float (&v)[8]) {
      float4* q = reinterpret_cast<float4*>(dst + o);
      float4 a = q[0], b = q[1];
      a.x += v[0]; a.y += v[1]; a.z += v[2]; a.w += v[3];
      b.x += v[4]; b.y += v[5]; b.z += v[6]; b.w += v[7];
      q[0] = a;
      q[1] = b;
    };
    if (d.dw_up) add8(d.dw_up, gu[c]);
    if (d.dw_gate) add8(d.dw_gate, gg[c]);
    if (d.dw_down) add8(d.dw_down, gd[c]);
  }
}

// ------------------------------------------------------------------ per token: dx
// The token's active neurons are listed first (pack slots of every tile, or
// the recomputed gate row of a routed token), then taken kBwDxBatch at a
// time with all their W_up / W_gate row loads in flight.
constexpr int kBwDxBatch = 8;
constexpr int kBwDxList = 8192;    // list capacity in LDS (d_ff of a routed token)

template <bool BF, int CH>
__global__ __launch_bounds__(kBwThreads) void k_bw_dx(const BwDesc d) {
  __shared__ int s_i[kBwDxList];
  __shared__ int s_scan[4];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int r = d.slot_of[t];
  const float b = bw_bias(d, t), cut = bw_cut(d, t);
  // ---- the list: neuron ids (the pair position follows from them)
  int n_all = 0;
  if (r < 0) {
    for (int j0 = 0; j0 < d.ntiles; j0 += kBwThreads) {
      const int j = j0 + threadIdx.x;
      const int n = j < d.ntiles ? min(d.cnt[(size_t)t * d.ntiles + j], d.E) : 0;
      int tot = 0;
      const int ex = block_excl_scan<kBwThreads>(n, s_scan, &tot);
      for (int q = 0; q < n; ++q) {
        const size_t pk = (size_t)t * d.ntiles + j;
        s_i[n_all + ex + q] = (int)(pk * d.E + q);          // pack position
      }
      n_all += tot;
    }
  } else {
    for (int i0 = 0; i0 < d.F; i0 += kBwThreads) {
      const int i = i0 + threadIdx.x;
      const bool on = i < d.F && d.zr[(size_t)r * d.F + i] + b > cut;
      int tot = 0;
      const int ex = block_excl_scan<kBwThreads>(on ? 1 : 0, s_scan, &tot);
      if (on) s_i[n_all + ex] = i;                            // neuron id
      n_all += tot;
    }
  }
  if (threadIdx.x == 0) s_n = n_all;
  __syncthreads();
  const int n = s_n;

  float acc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  // split S = gridDim.y of this token's list: batch b goes to split b mod S
  const int S = gridDim.y;
  for (int s0 = blockIdx.y * kBwDxBatch; s0 < n; s0 += S * kBwDxBatch) {
    Raw8<BF> wu[kBwDxBatch][CH], wg[kBwDxBatch][CH];
    float du[kBwDxBatch], dz[kBwDxBatch];
#pragma unroll
    for (int bb = 0; bb < kBwDxBatch; ++bb) {
      const bool live = s0 + bb < n;
      int i = 0;
      long long p = 0;
      if (live) {
        const int v = s_i[s0 + bb];
        if (r < 0) {
          p = v;
          const int pk = v / d.E;
          i = (pk % d.ntiles) * d.T + d.idx[p];
        } else {
          i = v;
          p = d.pbase + (long long)r * d.F + i;
        }
      }
      du[bb] = live ? d.du[p] : 0.f;
      dz[bb] = live ? d.dz[p] : 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int col = (threadIdx.x + c * kBwThreads) * 8;
        wu[bb][c].load(d.w_up, (size_t)i * d.d + col, live && col < d.d);
        wg[bb][c].load(d.w_gate, (size_t)i * d.d + col, live && col < d.d);
      }
    }
#pragma unroll
    for (int bb = 0; bb < kBwDxBatch; ++bb)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float a8[8], g8[8];
        wu[bb][c].get(a8);
        wg[bb][c].get(g8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = fmaf(dz[bb], g8[e], fmaf(du[bb], a8[e], acc[c][e]));
      }
  }
  if (S > 1) {
    // fp32 partial row of this split; k_bw_dxsum adds the splits in order
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = (threadIdx.x + c * kBwThreads) * 8;
      if (col >= d.d) continue;
      float* o = d.dxp + ((size_t)blockIdx.y * d.m + t) * d.d + col;
      *reinterpret_cast<float4*>(o) = float4{acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
      *reinterpret_cast<float4*>(o + 4) = float4{acc[c][4], acc[c][5], acc[c][6], acc[c][7]};
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = (threadIdx.x + c * kBwThreads) * 8;
    if (col >= d.d) continue;
    if constexpr (BF) {
      uint4 o;
      o.x = f2bf(acc[c][0]) | (f2bf(acc[c][1]) << 16);
      o.y = f2bf(acc[c][2]) | (f2bf(acc[c][3]) << 16);
      o.z = f2bf(acc[c][4]) | (f2bf(acc[c][5]) << 16);
      o.w = f2bf(acc[c][6]) | (f2bf(acc[c][7]) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(d.dx) + (size_t)t * d.d + col) = o;
    } else {
      float* o = static_cast<float*>(d.dx) + (size_t)t * d.d + col;
      *reinterpret_cast<float4*>(o) = float4{acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
      *reinterpret_cast<float4*>(o + 4) = float4{acc[c][4], acc[c][5], acc[c][6], acc[c][7]};
    }
  }
}

// dx of token blockIdx.x from its splits' fp32 partial rows, added in split order
__global__ __launch_bounds__(kBwThreads) void k_bw_dxsum(const BwDesc d, int S) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * kBwThreads + threadIdx.x) * 8;
  if (col >= d.d) return;
  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float* p = d.dxp + ((size_t)sp * d.m + t) * d.d + col;
    const float4 u = *reinterpret_cast<const float4*>(p), v = *reinterpret_cast<const float4*>(p + 4);
    a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w; a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
  }
  if (d.dtype == DT_BF16) {
    uint4 o;
    o.x = f2bf(a[0]) | (f2bf(a[1]) << 16);
    o.y = f2bf(a[2]) | (f2bf(a[3]) << 16);
    o.z = f2bf(a[4]) | (f2bf(a[5]) << 16);
    o.w = f2bf(a[6]) | (f2bf(a[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(d.dx) + (size_t)t * d.d + col) = o;
  } else {
    float* o = static_cast<float*>(d.dx) + (size_t)t * d.d + col;
    *reinterpret_cast<float4*>(o) = float4{a[0], a[1], a[2], a[3]};
    *reinterpret_cast<float4*>(o + 4) = float4{a[4], a[5], a[6], a[7]};
  }
}

// ------------------------------------------------------------------ launches
static bool bw_shape_ok(const BwDesc& d) {
  // the dx list holds a routed token's d_ff neurons, a compact token's
  // ntiles * E pack slots
  return d.m >= 1 && d.d % 8 == 0 && d.d <= 8 * kBwChunks * kBwThreads && d.T <= 1024 && d.F % d.T == 0 &&
         d.nblk == (d.m + kBwBlock - 1) / kBwBlock && (long long)d.ntiles * d.E <= kBwDxList &&
         (!d.routing || d.F <= kBwDxList);
}

// Row t of (du | dz): zero, then the token's active neurons (the same list
// as k_bw_dx), staged in LDS and written with 16-byte stores.
__global__ __launch_bounds__(kBwThreads) void k_bw_duz(const BwDesc d) {
  extern __shared__ uint4 s_dz4[];
  uint16_t* s_row = reinterpret_cast<uint16_t*>(s_dz4);      // [2F]
  const int t = blockIdx.x, F = d.F, n16 = 2 * F / 8;
  const int r = d.slot_of[t];
  for (int c = threadIdx.x; c < n16; c += kBwThreads) s_dz4[c] = uint4{0, 0, 0, 0};
  __syncthreads();
  if (r < 0) {
    const int nslots = d.ntiles * d.E;
    for (int q0 = threadIdx.x; q0 < nslots; q0 += kBwThreads) {
      const int j = q0 / d.E, q = q0 - j * d.E;
      const size_t pk = (size_t)t * d.ntiles + j;
      if (q < min(d.cnt[pk], d.E)) {
        const long long p = (long long)pk * d.E + q;
        const int i = j * d.T + d.idx[p];
        s_row[i] = (uint16_t)f2bf(d.du[p]);
        s_row[F + i] = (uint16_t)f2bf(d.dz[p]);
      }
    }
  } else {
    const float b = bw_bias(d, t), cut = bw_cut(d, t);
    for (int i = threadIdx.x; i < F; i += kBwThreads)
      if (d.zr[(size_t)r * F + i] + b > cut) {
        const long long p = d.pbase + (long long)r * F + i;
        s_row[i] = (uint16_t)f2bf(d.du[p]);
        s_row[F + i] = (uint16_t)f2bf(d.dz[p]);
      }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(d.duz + (size_t)t * 2 * F);
  for (int c = threadIdx.x; c < n16; c += kBwThreads) dst[c] = s_dz4[c];
}

hipError_t launch_bw_duz(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d) || !d.duz || d.dtype != DT_BF16 || d.F % 8 != 0) return hipErrorInvalidValue;
  const size_t lds = (size_t)d.F * 2 * sizeof(uint16_t);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  ffn_launch(k_bw_duz, dim3(d.m), dim3(kBwThreads), lds, s, d);
  return hipGetLastError();
}

hipError_t launch_bw_slots(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d)) return hipErrorInvalidValue;
  ffn_launch(k_bw_slots, dim3(1), dim3(1024), 0, s, d);
  return hipGetLastError();
}
hipError_t launch_bw_count(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d)) return hipErrorInvalidValue;
  ffn_launch(k_bw_count, dim3(d.ntiles, d.nblk), dim3(kBwThreads), 0, s, d);
  return hipGetLastError();
}
hipError_t launch_bw_scan(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d)) return hipErrorInvalidValue;
  ffn_launch(k_bw_offsets, dim3((d.F + kBwThreads - 1) / kBwThreads), dim3(kBwThreads), 0, s, d);
  ffn_launch(k_bw_colptr, dim3(1), dim3(1024), 0, s, d);
  return hipGetLastError();
}
hipError_t launch_bw_fill(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d)) return hipErrorInvalidValue;
  ffn_launch(k_bw_fill, dim3(d.ntiles, d.nblk), dim3(kBwThreads), 0, s, d);
  return hipGetLastError();
}
hipError_t launch_bw_neuron(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d)) return hipErrorInvalidValue;
  const bool two = d.d > 8 * kBwThreads;
  if (d.dtype == DT_BF16) {
    if (two) ffn_launch((k_bw_neuron<true, 2>), dim3(d.F), dim3(kBwThreads), 0, s, d);
    else ffn_launch((k_bw_neuron<true, 1>), dim3(d.F), dim3(kBwThreads), 0, s, d);
  } else {
    if (two) ffn_launch((k_bw_neuron<false, 2>), dim3(d.F), dim3(kBwThreads), 0, s, d);
    else ffn_launch((k_bw_neuron<false, 1>), dim3(d.F), dim3(kBwThreads), 0, s, d);
  }
  return hipGetLastError();
}
int bw_dx_splits(int m) { return std::max(1, std::min(kBwDxMaxSplit, kBwDxPartRows / std::max(m, 1))); }

hipError_t launch_bw_dx(const BwDesc& d, hipStream_t s) {
  if (!bw_shape_ok(d) || !d.dx) return hipErrorInvalidValue;
  const int S = bw_dx_splits(d.m);
  if (S > 1 && !d.dxp) return hipErrorInvalidValue;
  const bool two = d.d > 8 * kBwThreads;
  const dim3 grid(d.m, S);
  if (d.dtype == DT_BF16) {
    if (two) ffn_launch((k_bw_dx<true, 2>), grid, dim3(kBwThreads), 0, s, d);
    else ffn_launch((k_bw_dx<true, 1>), grid, dim3(kBwThreads), 0, s, d);
  } else {
    if (two) ffn_launch((k_bw_dx<false, 2>), grid, dim3(kBwThreads), 0, s, d);
    else ffn_launch((k_bw_dx<false, 1>), grid, dim3(kBwThreads), 0, s, d);
  }
  if (S > 1) ffn_launch(k_bw_dxsum, dim3(d.m, (d.d + 8 * kBwThreads - 1) / (8 * kBwThreads)), dim3(kBwThreads), 0, s, d, S);
  return hipGetLastError();
}

}  // namespace ffn
