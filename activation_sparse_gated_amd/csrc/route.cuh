// Routing of a TwELL pack, run by one workgroup of 256 threads at the end of
// the sparse pass (or on its own after a standalone gate pass).
#pragma once
#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

// ------------------------------------------------------------------ routing
// One workgroup (256 threads): route_t = any tile with cnt > E; dense_list =
// routed ids ascending; n_dense. Then advances the look-back epoch (the gate
// pass that wrote this pack has completed).
__device__ inline void route_pass(const RouteDesc& r) {
  __shared__ int s_over[1024];
  __shared__ int s_scan[4];
  int base = 0;
  for (int c0 = 0; c0 < r.M; c0 += 1024) {
    const int n = min(1024, r.M - c0);
    for (int i = threadIdx.x; i < 1024; i += blockDim.x) s_over[i] = 0;
    __syncthreads();
    // sixteen counts per thread in flight, then tested: one memory round per
    // 16 * blockDim counts instead of one per blockDim
    const int np = n * r.ntiles;
    const int32_t* cb = r.cnt + (size_t)c0 * r.ntiles;   // the chunk's tokens are consecutive rows
    for (int p0 = threadIdx.x; p0 < np; p0 += 16 * blockDim.x) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int p = p0 + u * blockDim.x;
        v[u] = p < np ? cb[p] : 0;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int p = p0 + u * blockDim.x;
        if (p < np && v[u] > r.E) s_over[p / r.ntiles] = 1;
      }
    }
    __syncthreads();
    int o[4], ro = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = threadIdx.x * 4 + i;
      o[i] = t < n ? s_over[t] : 0;
      ro += o[i];
    }
    int tot;
    int xo = block_excl_scan<256>(ro, s_scan, &tot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = threadIdx.x * 4 + i;
      if (t < n) {
        r.route[c0 + t] = (uint8_t)o[i];
        if (o[i]) r.dense_list[base + xo] = c0 + t;
        xo += o[i];
      }
    }
    base += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *r.n_dense = base;
    const uint32_t ep = __hip_atomic_load(&r.ctrl[CTRL_EPOCH], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&r.ctrl[CTRL_EPOCH], ep + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace ffn
