// Mixture-of-experts layer over sparse FFN experts: the two data-movement
// kernels around the experts' own forward passes. (LoPA page, "Model Casting
// and Quality at 90% Sparsity": the gating applies to MoE experts, which are
// FFN blocks.)
//
//   k_moe_gather   one workgroup per grouped row: the token's x row, and its
//                  routing slot's bias and threshold, into the expert-grouped
//                  buffers (experts' rows contiguous, tokens in order).
//   k_moe_combine  y[t] = sum over t's slots s, in slot order, of
//                  w[t, s] * y_grouped[pos(t, s)] (fp32), rounded once.
// The routing table is a kernel argument (at most kMoeMaxPairs pairs).
#include "common.cuh"
#include "kernels.cuh"

namespace ffn {

__global__ __launch_bounds__(256) void k_moe_gather(const MoeDesc d) {
  const int r = blockIdx.x;                         // grouped row
  const int ts = d.tab.src[r], t = ts / d.topk;
  const int esz = d.dtype == DT_BF16 ? 2 : 4;
  const size_t rowb = (size_t)d.d * esz;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(d.x) + (size_t)t * rowb);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(d.xg) + (size_t)r * rowb);
  for (int c = threadIdx.x; c < (int)(rowb / 16); c += blockDim.x) dst[c] = src[c];
  if (threadIdx.x == 0) {
    if (d.tau) d.tg[r] = d.tau[ts];
    if (d.bias) d.bg[r] = d.bias[ts];
  }
}

__global__ __launch_bounds__(256) void k_moe_combine(const MoeDesc d) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;     // column
  if (c >= d.d) return;
  float acc = 0.f;
  for (int s = 0; s < d.topk; ++s) {
    const int q = t * d.topk + s;
    const int row = d.tab.pos[q];
    const float w = d.tab.w[q];
    float v;
    if (d.dtype == DT_BF16)
      v = bf2f(static_cast<const uint16_t*>(d.yg)[(size_t)row * d.d + c]);
    else
      v = static_cast<const float*>(d.yg)[(size_t)row * d.d + c];
    acc = fmaf(w, v, acc);
  }
  if (d.dtype == DT_BF16)
    static_cast<uint16_t*>(d.y)[(size_t)t * d.d + c] = (uint16_t)f2bf(acc);
  else
    static_cast<float*>(d.y)[(size_t)t * d.d + c] = acc;
}

hipError_t launch_moe_gather(const MoeDesc& d, hipStream_t s) {
  if (d.npairs < 1 || d.npairs > kMoeMaxPairs || d.d % 8 != 0) return hipErrorInvalidValue;
  ffn_launch(k_moe_gather, dim3(d.npairs), dim3(256), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const MoeDesc& d, hipStream_t s) {
  if (d.m < 1 || d.m * d.topk > kMoeMaxPairs || d.m > 65535) return hipErrorInvalidValue;
  ffn_launch(k_moe_combine, dim3((d.d + 255) / 256, d.m), dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace ffn
