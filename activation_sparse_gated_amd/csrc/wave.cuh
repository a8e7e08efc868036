// Wave-level helpers shared by the decode and prefill kernels: the transpose
// reduction of several values across a wave and 8-element dot products.
#pragma once
#include "common.cuh"

namespace ffn {

// ------------------------------------------------------------------ wave transpose reduction
// Reduces N values per lane across the 64 lanes of a wave. Each halving step
// keeps one half of the values and swaps the other half with the partner lane
// (wave_xchg: DPP inside a 16-lane row, ds_bpermute across rows), so
// N - 1 + (6 - log2 N) exchanges replace N full butterflies. Afterwards v[0]
// of lane L holds the wave total of value index L >> (6 - log2 N).
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
      v[j] = keep + wave_xchg<O>(send);
    }
    WaveTRed<N / 2, O / 2>::run(v, lane);
  }
};
template <int O>
struct WaveTRed<1, O> {
  template <int V>
  __device__ __forceinline__ static void run(float (&v)[V], int lane) {
    v[0] += wave_xchg<O>(v[0]);
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
// the same dot with v_dot2c_f32_bf16: pairs of bf16 products accumulated in
// fp32, four instructions per 8 elements and no unpacking
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_bf_d2(const uint4 a, const uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
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

}  // namespace ffn
