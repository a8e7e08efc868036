// Fused sparse up + down projection over the TwELL pack.
//
// For every packed neuron i of a non-routed token t: u_i = <W_up[i, :], x_t>,
// h_i = a_i * u_i (top-k packs already hold h_i), y_t += h_i * W_down[:, i].
// Both weight rows are contiguous (W_up is neuron-major already, W_down is
// kept neuron-major in the workspace), so a wave gathers each one with 16-byte
// loads that cover 1 KB contiguous per instruction. h never leaves registers:
// the up dot product is reduced across the wave by butterfly and immediately
// scales the down row. [Sparser/Faster/Lighter page (news.neo-ai.one,
// "Sparser, Faster, Lighter Transformer Language Models"), section
// "TwELL 減掉轉換開銷": one pass computes up and down without storing h.]
//
// Work split: the packed entries of all non-routed tokens form one list in
// (token, tile, slot) order; workgroup b takes a contiguous chunk of it. A
// token whose entries fall inside one chunk gets its y row written directly;
// a token spread over several chunks leaves one fp32 partial row per chunk,
// summed by k_ud_reduce in chunk order (deterministic).
#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

constexpr int UD_WAVES = 4;

template <int DT>
struct ElemTraits;
template <>
struct ElemTraits<DT_BF16> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  __device__ static void to_f32(const uint4 v, float* f) { unpack8(v, f); }
  __device__ static float scalar(const void* p, size_t i) { return bf2f(reinterpret_cast<const uint16_t*>(p)[i]); }
};
template <>
struct ElemTraits<DT_F32> {
  static constexpr int EPC = 4;
  __device__ static void to_f32(const uint4 v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static float scalar(const void* p, size_t i) { return reinterpret_cast<const float*>(p)[i]; }
};

__device__ __forceinline__ int ud_chunk(const UpdownDesc& u, int ntot) {
  return max(u.min_chunk, (ntot + u.grid - 1) / u.grid);
}

// first token t with offs[t + 1] > pos (offs is non-decreasing, offs[M] > pos)
__device__ __forceinline__ int token_of(const int32_t* offs, int M, int pos) {
  int lo = 0, hi = M - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (offs[mid + 1] > pos) hi = mid; else lo = mid + 1;
  }
  return lo;
}

template <int CPL, int DT>
__global__ __launch_bounds__(256) void k_updown(const UpdownDesc u) {
  using TR = ElemTraits<DT>;
  constexpr int EPC = TR::EPC;
  constexpr int VPL = CPL * EPC;                  // values per lane
  __shared__ int s_tp[1025];                      // per-token tile prefix of cnt
  __shared__ float s_y[UD_WAVES][CPL * 64 * EPC];
  __shared__ int s_scan[4];
  const int M = u.M, d = u.d, T = u.T, E = u.E;
  const int ntiles = u.F / T, nch = d / EPC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntot = min(u.offs[M], M * (u.F < 1 ? 1 : u.F));
  if (ntot <= 0) return;
  const int chunk = ud_chunk(u, ntot);
  const int b = blockIdx.x;
  int start = b * chunk;
  if (start >= ntot) return;
  const int end = min(start + chunk, ntot);
  int t = token_of(u.offs, M, start);

  while (start < end) {
    while (t < M - 1 && u.offs[t + 1] <= start) ++t;   // skip tokens without entries
    const int n0 = u.offs[t], n1 = u.offs[t + 1];
    if (n1 <= start) break;                        // malformed schedule: stop
    const int seg_end = min(end, n1);
    const int p0 = start - n0, p1 = seg_end - n0;

    // exclusive prefix of this token's tile counts
    {
      int total;
      for (int c0 = 0; c0 < ntiles; c0 += 256) {
        const int j = c0 + threadIdx.x;
        const int c = j < ntiles ? u.cnt[(size_t)t * ntiles + j] : 0;
        const int base = c0 == 0 ? 0 : s_tp[c0];
        __syncthreads();
        const int ex = block_excl_scan<256>(c, s_scan, &total);
        if (j < ntiles) s_tp[j] = base + ex;
        if (threadIdx.x == 0) s_tp[min(c0 + 256, ntiles)] = base + total;
        __syncthreads();
      }
    }

    float xr[VPL], ya[VPL];
    const size_t xrow = (size_t)t * d;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      float f[EPC];
      if (c < nch && !u.down_only) TR::to_f32(ldg16((const char*)u.x + (xrow + (size_t)c * EPC) * (DT == DT_BF16 ? 2 : 4)), f);
      else for (int q = 0; q < EPC; ++q) f[q] = 0.f;
#pragma unroll
      for (int q = 0; q < EPC; ++q) { xr[i * EPC + q] = f[q]; ya[i * EPC + q] = 0.f; }
    }

    const size_t esz = DT == DT_BF16 ? 2 : 4;
    for (int p = p0 + wave; p < p1; p += UD_WAVES) {
      int lo = 0, hi = ntiles - 1;                 // tile j with s_tp[j] <= p < s_tp[j + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tp[mid] <= p) lo = mid; else hi = mid - 1;
      }
      const int j = lo, slot = p - s_tp[j];
      const size_t ent = ((size_t)t * ntiles + j) * E + slot;
      const int neuron = j * T + u.idx[ent];
      const float a = TR::scalar(u.val, ent);
      const char* up = (const char*)u.w_up + (size_t)neuron * d * esz;
      const char* dn = (const char*)u.w_down_nm + (size_t)neuron * d * esz;
      uint4 ur[CPL], dr[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        const bool ok = c < nch;
        ur[i] = (ok && !u.down_only) ? ldg16(up + (size_t)c * 16) : uint4{0, 0, 0, 0};
        dr[i] = ok ? ldg16(dn + (size_t)c * 16) : uint4{0, 0, 0, 0};
      }
      float h = a;
      if (!u.down_only) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          float f[EPC];
          TR::to_f32(ur[i], f);
#pragma unroll
          for (int q = 0; q < EPC; ++q) s = fmaf(f[q], xr[i * EPC + q], s);
        }
        h = a * wave_sum(s);
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float f[EPC];
        TR::to_f32(dr[i], f);
#pragma unroll
        for (int q = 0; q < EPC; ++q) ya[i * EPC + q] = fmaf(h, f[q], ya[i * EPC + q]);
      }
    }

    // combine the waves in a fixed order
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < EPC; ++q) s_y[wave][(i * 64 + lane) * EPC + q] = ya[i * EPC + q];
    __syncthreads();
    const bool whole = (n0 / chunk) == ((n1 - 1) / chunk);
    for (int e = threadIdx.x; e < d; e += 256) {
      const int cidx = e / EPC, q = e % EPC;      // element e lives in chunk cidx, slot q
      const int ii = cidx / 64, ln = cidx % 64;
      const int o = (ii * 64 + ln) * EPC + q;
      const float s = ((s_y[0][o] + s_y[1][o]) + s_y[2][o]) + s_y[3][o];
      if (whole) {
        if (DT == DT_BF16) reinterpret_cast<uint16_t*>(u.y)[(size_t)t * d + e] = (uint16_t)f2bf(s);
        else reinterpret_cast<float*>(u.y)[(size_t)t * d + e] = s;
      } else {
        u.partial[(size_t)(b + t) * d + e] = s;
      }
    }
    __syncthreads();
    start = seg_end;
    ++t;
  }
}

// y rows of non-routed tokens: zero when the token has no entry, the ordered
// sum of its chunk partials when its entries span several workgroups.
template <int DT>
__global__ __launch_bounds__(256) void k_ud_reduce(const UpdownDesc u) {
  __shared__ float s_red[4][64];
  const int t = blockIdx.y, d = u.d;
  const int e = blockIdx.x * 64 + (threadIdx.x & 63), grp = threadIdx.x >> 6;
  if (u.route[t]) return;
  const int n0 = u.offs[t], n1 = u.offs[t + 1];
  float s = 0.f;
  if (n1 > n0) {
    const int chunk = ud_chunk(u, u.offs[u.M]);
    const int blo = n0 / chunk, bhi = (n1 - 1) / chunk;
    if (blo == bhi) return;                        // written by the sparse kernel
    if (e < d)
      for (int b = blo + grp; b <= bhi; b += 4) s += u.partial[(size_t)(b + t) * d + e];
  }
  s_red[grp][threadIdx.x & 63] = s;
  __syncthreads();
  if (grp == 0 && e < d) {
    const int l = threadIdx.x;
    const float v = ((s_red[0][l] + s_red[1][l]) + s_red[2][l]) + s_red[3][l];
    if (DT == DT_BF16) reinterpret_cast<uint16_t*>(u.y)[(size_t)t * d + e] = (uint16_t)f2bf(v);
    else reinterpret_cast<float*>(u.y)[(size_t)t * d + e] = v;
  }
}

template <int DT>
static hipError_t go_updown(const UpdownDesc& u, hipStream_t s) {
  const int epc = DT == DT_BF16 ? 8 : 4;
  const int cpl = (u.d / epc + 63) / 64;
  dim3 grid(u.grid);
  switch (cpl) {
    case 1: hipLaunchKernelGGL((k_updown<1, DT>), grid, dim3(256), 0, s, u); break;
    case 2: hipLaunchKernelGGL((k_updown<2, DT>), grid, dim3(256), 0, s, u); break;
    case 3:
    case 4: hipLaunchKernelGGL((k_updown<4, DT>), grid, dim3(256), 0, s, u); break;
    case 5: case 6: case 7:
    case 8: hipLaunchKernelGGL((k_updown<8, DT>), grid, dim3(256), 0, s, u); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_updown(const UpdownDesc& u, hipStream_t s) {
  if (u.M <= 0) return hipSuccess;
  return u.dtype == DT_BF16 ? go_updown<DT_BF16>(u, s) : go_updown<DT_F32>(u, s);
}

hipError_t launch_updown_reduce(const UpdownDesc& u, hipStream_t s) {
  if (u.M <= 0) return hipSuccess;
  dim3 grid((u.d + 63) / 64, u.M);
  if (u.dtype == DT_BF16) hipLaunchKernelGGL(k_ud_reduce<DT_BF16>, grid, dim3(256), 0, s, u);
  else hipLaunchKernelGGL(k_ud_reduce<DT_F32>, grid, dim3(256), 0, s, u);
  return hipGetLastError();
}

}  // namespace ffn
