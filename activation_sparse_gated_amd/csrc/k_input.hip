// Input-side selection of the gate projection (bf16): per token, keep the
// k_in input channels j with the largest |x_j| * ||W[:, j]||_2 and read only
// their weights (WINA page, section 3.1, applied to the gate's input: the
// score of an input element is its magnitude times the norm of the weight
// column it multiplies; with equal norms it is section 二's |x| rule).
//
// The gate input matrix W (W_gate [F x d], or V [r x d] of a low-rank gate)
// is kept input-major, W^T [d x N], so one kept channel's weights are one
// contiguous row of N values. Three kernels:
//   k_in_select  one workgroup per token: scores in fp32 (c is correctly
//                rounded), the k_in-th largest found by a four-pass 8-bit
//                radix select on the score bits, ties taken in index order;
//                the kept channels ascending with their x values
//   k_in_gemv    partial[g][t][n] = sum over the kept channels of group g of
//                x_j W^T[j, n]: workgroups over (512-column slices x channel
//                groups x tokens), a lane holding 8 columns, the waves' sums
//                added in LDS in wave order
//   k_in_pack    full gate: g = sum of the group partials in group order, the
//                selection z = g + b > cut, and the TwELL pack of one
//                (token, tile) per workgroup (no look-back: the workgroup owns
//                the tile); a low-rank gate instead adds the partials into t
//                (k_in_sum) and continues with U t
#include <algorithm>

#include "common.cuh"
#include "kernels.cuh"
#include "wave.cuh"

namespace ffn {

constexpr int kInSelThreads = 1024;
constexpr int kInGemvWaves = 16;
constexpr int kInMaxPerWave = 8;          // kept channels a wave of k_in_gemv holds in flight

// ------------------------------------------------------------------ k_in_select
__global__ __launch_bounds__(kInSelThreads) void k_in_select(const InDesc d) {
  __shared__ int s_hist[256];
  __shared__ int s_scan[kInSelThreads / 64];
  __shared__ uint32_t s_digit;
  __shared__ int s_rank;
  const int tid = threadIdx.x, t = blockIdx.x;
  const int dm = d.d, k = d.k;
  if (k <= 0) return;
  const uint16_t* xt = reinterpret_cast<const uint16_t*>(d.x) + (size_t)t * dm;
  // thread tid holds channels 4 tid .. 4 tid + 3 (index order = thread order)
  uint32_t key[4];
  uint16_t xb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 4 * tid + q;
    xb[q] = j < dm ? xt[j] : (uint16_t)0;
    key[q] = j < dm ? __float_as_uint(fabsf(bf2f(xb[q])) * d.colnorm[j]) : 0u;   // s >= 0: bit order = value order
  }
  // the k-th largest key, 8 bits at a time from the top; kk = its rank among
  // the keys that share the prefix found so far
  uint32_t prefix = 0u, mask = 0u;
  int kk = k;
  for (int pass = 3; pass >= 0; --pass) {
    const int shift = pass * 8;
    for (int i = tid; i < 256; i += kInSelThreads) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * tid + q < dm && (key[q] & mask) == prefix) atomicAdd(&s_hist[(key[q] >> shift) & 255u], 1);
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255 - 4 l .. 252 - 4 l (high to low); counts above
      // each digit by an inclusive scan over the lanes
      int c[4], loc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = s_hist[255 - 4 * tid - e];
        loc += c[e];
      }
      const int incl = wave_incl_scan(loc);
      int above = incl - loc;                        // keys with a higher digit than this lane's first
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < kk && kk <= above + c[e]) {
          s_digit = 255u - (uint32_t)(4 * tid + e);
          s_rank = kk - above;
        }
        above += c[e];
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    kk = s_rank;
    __syncthreads();
  }
  // keep key > prefix, and the first kk keys equal to it in index order
  int tie[4], nt = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    tie[q] = (4 * tid + q < dm && key[q] == prefix) ? 1 : 0;
    nt += tie[q];
  }
  int tot;
  int trank = block_excl_scan<kInSelThreads>(nt, s_scan, &tot);
  int sel[4], ns = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool gt = 4 * tid + q < dm && key[q] > prefix;
    sel[q] = (gt || (tie[q] && trank < kk)) ? 1 : 0;
    trank += tie[q];
    ns += sel[q];
  }
  int pos = block_excl_scan<kInSelThreads>(ns, s_scan, &tot);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (sel[q]) {
      d.kidx[(size_t)t * k + pos] = 4 * tid + q;
      d.kval[(size_t)t * k + pos] = xb[q];
      ++pos;
    }
}

// ------------------------------------------------------------------ k_in_gemv
__global__ __launch_bounds__(64 * kInGemvWaves) void k_in_gemv(const InDesc d) {
  __shared__ float s_acc[kInGemvWaves][512];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int S = (d.N + 511) / 512;
  const int slice = blockIdx.x % S, grp = blockIdx.x / S, t = blockIdx.y;
  const int col = slice * 512 + lane * 8;
  const int cpg = (d.k + d.groups - 1) / d.groups;
  const int p0 = grp * cpg, p1 = min(d.k, p0 + cpg);
  // this wave's channels p0 + wave, p0 + wave + 16, ...: ids first, then rows
  int jj[kInMaxPerWave];
  float xv[kInMaxPerWave];
#pragma unroll
  for (int i = 0; i < kInMaxPerWave; ++i) {
    const int p = p0 + wave + i * kInGemvWaves;
    const bool on = p < p1;
    jj[i] = on ? d.kidx[(size_t)t * d.k + p] : -1;
    xv[i] = on ? bf2f(d.kval[(size_t)t * d.k + p]) : 0.f;
  }
  uint4 w[kInMaxPerWave];
#pragma unroll
  for (int i = 0; i < kInMaxPerWave; ++i)
    w[i] = (jj[i] >= 0 && col < d.N) ? ldg16(d.wt + (size_t)jj[i] * d.N + col) : uint4{0, 0, 0, 0};
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kInMaxPerWave; ++i) {
    float f[8];
    unpack8(w[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(xv[i], f[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_acc[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < 512) {
    const int c = slice * 512 + (int)threadIdx.x;
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < kInGemvWaves; ++wv) s += s_acc[wv][threadIdx.x];
    if (c < d.N) d.part[((size_t)grp * d.M + t) * d.N + c] = s;
  }
}

// Sum of the channel groups' partials of output element o (token-major index
// t N + n), in group order, 16 loads in flight at a time.
__device__ __forceinline__ float group_sum(const InDesc& d, size_t o) {
  const size_t stride = (size_t)d.M * d.N;
  float g = 0.f;
  for (int g0 = 0; g0 < d.groups; g0 += 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = g0 + i < d.groups ? d.part[(size_t)(g0 + i) * stride + o] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (g0 + i < d.groups) g += v[i];
  }
  return g;
}

// ------------------------------------------------------------------ k_in_sum
// Low-rank gate: t = the groups' partials summed in group order, into the
// first group's slab.
__global__ __launch_bounds__(256) void k_in_sum(const InDesc d) {
  const size_t o = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= (size_t)d.M * d.N) return;
  d.part[o] = group_sum(d, o);
}

// ------------------------------------------------------------------ k_in_pack
constexpr int kInPackThreads = 256;

__global__ __launch_bounds__(kInPackThreads) void k_in_pack(const InDesc d) {
  __shared__ int s_cnt[16];
  __shared__ int s_total;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int j = blockIdx.x, t = blockIdx.y, T = d.T, E = d.E;
  const int ntiles = d.N / T, nch = T / 64;        // 64-neuron chunks of the tile (T <= 1024)
  const float b = d.bias ? d.bias[t] : d.bias_scalar;
  const float cut = d.sel == SEL_THRESH ? fmaxf(d.tau[t], 0.f) : 0.f;
  // each wave takes chunks wave, wave + 4, ...: g (group partials in order), mask
  float z[4];
  uint64_t bal[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = wave + 4 * i;
    z[i] = 0.f;
    bal[i] = 0ull;
    if (ch < nch) {
      const int n = j * T + ch * 64 + lane;
      const float g = group_sum(d, (size_t)t * d.N + n);
      if (d.g_debug) d.g_debug[(size_t)t * d.N + n] = g;
      z[i] = g + b;
      bal[i] = ballot64(z[i] > cut);
      if (lane == 0) s_cnt[ch] = __popcll(bal[i]);
    }
  }
  __syncthreads();
  const size_t slot0 = ((size_t)t * ntiles + j) * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = wave + 4 * i;
    if (ch < nch) {
      int pre = 0;
      for (int c = 0; c < ch; ++c) pre += s_cnt[c];
      const int pos = pre + __popcll(bal[i] & lanemask_lt());
      if (((bal[i] >> lane) & 1ull) && pos < E) {
        d.idx[slot0 + pos] = (uint16_t)(ch * 64 + lane);
        reinterpret_cast<uint16_t*>(d.val)[slot0 + pos] = (uint16_t)f2bf(z[i]);
      }
    }
  }
  if (threadIdx.x == 0) {
    int total = 0;
    for (int c = 0; c < nch; ++c) total += s_cnt[c];
    s_total = total;
  }
  __syncthreads();
  const int total = s_total;
  if (threadIdx.x == 0) d.cnt[(size_t)t * ntiles + j] = total;
  for (int s = min(total, E) + (int)threadIdx.x; s < E; s += kInPackThreads) {
    d.idx[slot0 + s] = 0xFFFF;
    reinterpret_cast<uint16_t*>(d.val)[slot0 + s] = 0;
  }
}

// ------------------------------------------------------------------ launches
// Channel groups: about 256 workgroups in all, but at most 32 groups (each
// output then sums at most 32 partials), and at least enough that a group
// fits the waves' loads.
int in_groups(int N, int k) {
  const int S = (N + 511) / 512;
  int g = std::max(1, std::min(32, 256 / S));
  g = std::min(g, std::max(1, k));
  while ((k + g - 1) / g > kInGemvWaves * kInMaxPerWave) ++g;
  return g;
}

bool in_ok(const InDesc& d) {
  if (d.M < 1 || d.d < 8 || d.d > 4 * kInSelThreads || d.k < 0 || d.k > d.d || d.N < 8 || d.N % 8 != 0) return false;
  if (d.groups < 1 || (d.k + d.groups - 1) / d.groups > kInGemvWaves * kInMaxPerWave) return false;
  return d.x && d.colnorm && d.kidx && d.kval && d.wt && d.part;
}

hipError_t launch_in_select(const InDesc& d, hipStream_t s) {
  if (!in_ok(d)) return hipErrorInvalidValue;
  ffn_launch(k_in_select, dim3(d.M), dim3(kInSelThreads), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_in_gemv(const InDesc& d, hipStream_t s) {
  if (!in_ok(d)) return hipErrorInvalidValue;
  const int S = (d.N + 511) / 512;
  ffn_launch(k_in_gemv, dim3(S * d.groups, d.M), dim3(64 * kInGemvWaves), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_in_sum(const InDesc& d, hipStream_t s) {
  if (!in_ok(d)) return hipErrorInvalidValue;
  const size_t n = (size_t)d.M * d.N;
  ffn_launch(k_in_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_in_pack(const InDesc& d, hipStream_t s) {
  if (!in_ok(d) || d.T < 64 || d.T % 64 != 0 || d.T > 1024 || d.N % d.T != 0 || d.E < 0 || d.E > d.T || !d.cnt ||
      !d.idx || !d.val)
    return hipErrorInvalidValue;
  ffn_launch(k_in_pack, dim3(d.N / d.T, d.M), dim3(kInPackThreads), 0, s, d);
  return hipGetLastError();
}

}  // namespace ffn
