// Set-up kernels: W_down layout change, WINA column norms, buffer fill.
#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

// dst[c][r] = src[r][c] through a 64 x 64 LDS tile (coalesced on both sides);
// dst rows are ldd elements apart.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, T* __restrict__ dst,
                                                  int rows, int cols, int ldd) {
  __shared__ T buf[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) buf[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[(size_t)c * ldd + r] = buf[tx][i];
  }
}

hipError_t launch_transpose_ld(const void* src, void* dst, int rows, int cols, int ldd, int esize, hipStream_t s) {
  if (ldd < rows) return hipErrorInvalidValue;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  if (esize == 2)
    ffn_launch(k_transpose<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src, (uint16_t*)dst, rows, cols, ldd);
  else
    ffn_launch(k_transpose<float>, grid, dim3(256), 0, s, (const float*)src, (float*)dst, rows, cols, ldd);
  return hipGetLastError();
}
hipError_t launch_transpose(const void* src, void* dst, int rows, int cols, int esize, hipStream_t s) {
  return launch_transpose_ld(src, dst, rows, cols, rows, esize, s);
}

// One wave per neuron row of the neuron-major W_down^T [F x d]: the column
// norm ||W_down[:, i]||_2 of the WINA score (WINA page, section 3.1). Each
// lane sums the squares of its strided elements in order, the wave combines
// them by butterfly, and the square root is taken in double, which rounds the
// fp32 result correctly.
__global__ __launch_bounds__(256) void k_rownorm(const void* __restrict__ w, float* __restrict__ c,
                                                 int F, int d, int dtype) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= F) return;
  float s = 0.f;
  if (dtype == DT_BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(w) + (size_t)row * d;
    for (int k = lane; k < d; k += 64) {
      const float v = bf2f(p[k]);
      s = fmaf(v, v, s);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(w) + (size_t)row * d;
    for (int k = lane; k < d; k += 64) s = fmaf(p[k], p[k], s);
  }
  s = wave_sum(s);
  if (lane == 0) c[row] = (float)sqrt((double)s);
}

hipError_t launch_rownorm(const void* w, float* c, int F, int d, int dtype, hipStream_t s) {
  ffn_launch(k_rownorm, dim3((F + 3) / 4), dim3(256), 0, s, w, c, F, d, dtype);
  return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// slab[0][i] = sum over z of slab[z][i], added in slab order (the low-rank
// first stage's split-K slabs, collapsed once before the gate GEMM reads t).
__global__ __launch_bounds__(256) void k_slab_sum(float* slabs, int nslabs, size_t stride, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = slabs[i];
  for (int z = 1; z < nslabs; ++z) s += slabs[(size_t)z * stride + i];
  slabs[i] = s;
}

hipError_t launch_slab_sum(float* slabs, int nslabs, size_t stride, size_t n, hipStream_t s) {
  if (nslabs <= 1 || n == 0) return hipSuccess;
  ffn_launch(k_slab_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, slabs, nslabs, stride, n);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  ffn_launch(k_fill_u32, dim3(blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

// TwELL pack from stored gate values (the masked dense sequence): wave w of
// the grid takes (token, tile) = (w / ntiles, w % ntiles) and walks the tile
// 64 neurons at a time. A neuron is active when z = g + b exceeds the cut
// (max(tau, 0) for a threshold, 0 for a bias); its slot is the count of
// active neurons before it in the tile (ballot prefix), kept while below E.
// [Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷": the tile-wise ELL layout.]
__global__ __launch_bounds__(256) void k_pack_g(const PackGDesc d) {
  const int lane = threadIdx.x & 63;
  const int ntiles = d.F / d.T;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long long)d.M * ntiles) return;                 // whole waves
  const int tok = (int)(w / ntiles), j = (int)(w - (long long)tok * ntiles);
  const float b = d.bias ? d.bias[tok] : d.bias_scalar;
  const float cut = d.sel == SEL_THRESH ? fmaxf(d.tau[tok], 0.f) : 0.f;
  const float* gr = d.g + (size_t)tok * d.F + (size_t)j * d.T;
  const size_t slot0 = ((size_t)tok * ntiles + j) * d.E;
  int run = 0;
  for (int c0 = 0; c0 < d.T; c0 += 64) {
    const int r = c0 + lane;
    float z = 0.f;
    bool act = false;
    if (r < d.T) {
      z = gr[r] + b;
      act = z > cut;
    }
    const uint64_t bal = ballot64(act);
    const int pos = run + __popcll(bal & lanemask_lt());
    if (act && pos < d.E) {
      d.idx[slot0 + pos] = (uint16_t)r;
      if (d.out_f32) reinterpret_cast<float*>(d.val)[slot0 + pos] = z;
      else reinterpret_cast<uint16_t*>(d.val)[slot0 + pos] = (uint16_t)f2bf(z);
    }
    run += __popcll(bal);
  }
  if (lane == 0) d.cnt[(size_t)tok * ntiles + j] = run;
  for (int sl = min(run, d.E) + lane; sl < d.E; sl += 64) {
    d.idx[slot0 + sl] = 0xFFFF;
    if (d.out_f32) reinterpret_cast<float*>(d.val)[slot0 + sl] = 0.f;
    else reinterpret_cast<uint16_t*>(d.val)[slot0 + sl] = 0;
  }
}

hipError_t launch_pack_g(const PackGDesc& d, hipStream_t s) {
  if (d.M <= 0) return hipSuccess;
  if (d.T <= 0 || d.T > 65535 || d.F % d.T != 0 || d.E < 0 || !d.g || !d.cnt || !d.idx || !d.val ||
      (d.sel == SEL_THRESH && !d.tau))
    return hipErrorInvalidValue;
  const long long waves = (long long)d.M * (d.F / d.T);
  ffn_launch(k_pack_g, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace ffn
